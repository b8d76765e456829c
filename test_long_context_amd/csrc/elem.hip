// Row-wise and elementwise kernels of the TTT-E2E path: embedding gather,
// RMSNorm forward/backward, RoPE application + key/value store scatter, the
// RoPE backward that packs dQKV, the fused vocabulary softmax-CE with its
// logit gradient, and small helpers. All are HBM-bound; they read and write
// each element once, with 16-byte accesses where the layout allows.
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace ttt {

static constexpr int RB = 256;  // threads per row-block

__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) sh[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += sh[i];
  return t;
}

// --------------------------------------------------------------- embedding
template <typename T>
__global__ void embed_kernel(const int32_t* tok, int n, const T* E, int d, float* h, int V, int* err) {
  const int t = blockIdx.x;
  const int id = tok[t];
  const bool ok = id >= 0 && id < V;
  if (!ok && threadIdx.x == 0) atomicOr(err, 1);
  for (int j = threadIdx.x; j < d; j += blockDim.x)
    h[(long)t * d + j] = ok ? to_f(E[(long)id * d + j]) : 0.f;
}

hipError_t embed_gather(DT dt, const int32_t* tok, int n, const void* E, int d, float* h, int V,
                        int* err, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (dt == DT::BF16)
    hipLaunchKernelGGL(embed_kernel<bf16>, dim3(n), dim3(RB), 0, st, tok, n, (const bf16*)E, d, h, V, err);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(n), dim3(RB), 0, st, tok, n, (const float*)E, d, h, V, err);
  return hipGetLastError();
}

// ----------------------------------------------------------------- RMSNorm
// Rows of up to RMS_MAXV float4 chunks per thread (d <= 4 RB RMS_MAXV).
static constexpr int RMS_MAXV = 8;

template <typename T>
__device__ __forceinline__ void store4(T* p, float4 v);
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, float4 v) {
  bf16x4 w;
  w[0] = (bf16)v.x;
  w[1] = (bf16)v.y;
  w[2] = (bf16)v.z;
  w[3] = (bf16)v.w;
  *(bf16x4*)p = w;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, float4 v) {
  *(float4*)p = v;
}
__device__ __forceinline__ float4 f4add(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }

// Row-sum of a float4 chunk set: a[i] += sum_p src[p * stride][chunk i]
// for p < np, the loads of four partials issued together before any add
// (one memory round trip per four partials, not one per load).
// 4 consecutive partial values at vector index v (float or bf16 storage)
__device__ __forceinline__ float4 ld_part4(const float* p, int v) { return ((const float4*)p)[v]; }
// raw 4-element loads and their conversion, for code that loads several
// parts before it uses any
__device__ __forceinline__ float4 ld_raw4(const float* p, int v) { return ((const float4*)p)[v]; }
__device__ __forceinline__ bf16x4 ld_raw4(const bf16* p, int v) { return ((const bf16x4*)p)[v]; }
__device__ __forceinline__ float4 raw_f4(float4 h) { return h; }
__device__ __forceinline__ float4 raw_f4(bf16x4 h) { return make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]); }
__device__ __forceinline__ float4 ld_part4(const bf16* p, int v) {
  const bf16x4 h = ((const bf16x4*)p)[v];
  return make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
}

// Loads take a clamped (valid) index and are unconditional: under a lane
// condition each becomes a branch with its own wait for memory; only the
// arithmetic and the stores check v < nv.
template <int NVT, typename PT = float>
__device__ __forceinline__ void rms_add_parts(float4 (&a)[NVT], const PT* src, long stride, int np, long row,
                                              int nv) {
  int p = 0;
  // the first group of up to four parts in straight-line code, so their
  // loads go out together with the caller's (a loop header in between
  // makes the caller's loads land before these are requested)
  {
    decltype(ld_raw4(src, 0)) t[4][NVT];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u < np)  // uniform
#pragma unroll
        for (int i = 0; i < NVT; ++i) t[u][i] = ld_raw4(src + u * stride + row, min((int)threadIdx.x + i * RB, nv - 1));
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u < np)
#pragma unroll
        for (int i = 0; i < NVT; ++i)
          if (threadIdx.x + i * RB < nv) a[i] = f4add(a[i], raw_f4(t[u][i]));
    p = np < 4 ? np : 4;
  }
  for (; p + 4 <= np; p += 4) {
    float4 t[4][NVT];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < NVT; ++i) {
        const int v = min((int)threadIdx.x + i * RB, nv - 1);
        t[u][i] = ld_part4(src + (p + u) * stride + row, v);
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < NVT; ++i)
        if (threadIdx.x + i * RB < nv) a[i] = f4add(a[i], t[u][i]);
  }
  for (; p < np; ++p) {
    float4 t[NVT];
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
      const int v = min((int)threadIdx.x + i * RB, nv - 1);
      t[i] = ld_part4(src + p * stride + row, v);
    }
#pragma unroll
    for (int i = 0; i < NVT; ++i)
      if (threadIdx.x + i * RB < nv) a[i] = f4add(a[i], t[i]);
  }
}

// x = x_in + sum_p parts[p] (pending split-K residual updates); x_out and
// save (either may be null) receive x; y = g * x * r with r = rsqrt(mean x^2 + eps).
// One workgroup per row; thread t holds float4 chunks t, t + RB, ... (NVT of
// them, d <= 4 RB NVT) in registers between the reduction and the output
// pass; the gain is requested with the row.
template <typename T, int NVT, typename PT>
__global__ void __launch_bounds__(RB) rms_fwd_kernel(const float* x_in, const PT* parts, int nsplit, long pstride,
                                                     float* x_out, float* save, const float* g, int d, float eps,
                                                     T* y, float* r) {
  __shared__ float sh[RB / 64];
  const long t = blockIdx.x;
  const int nv = d / 4;
  float4 xv[NVT], gv[NVT];
#pragma unroll
  for (int i = 0; i < NVT; ++i) {
    const int v = min((int)threadIdx.x + i * RB, nv - 1);
    xv[i] = ((const float4*)(x_in + t * d))[v];
    gv[i] = ((const float4*)g)[v];
  }
  rms_add_parts<NVT>(xv, parts, pstride, nsplit, t * d, nv);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NVT; ++i)
    if (threadIdx.x + i * RB < nv) {
      const float4 a = xv[i];
      ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    }
  ss = block_sum(ss, sh);
  const float rr = rsqrtf(ss / d + eps);
#pragma unroll
  for (int i = 0; i < NVT; ++i) {
    const int v = threadIdx.x + i * RB;
    if (v < nv) {
      const float4 a = xv[i], gg = gv[i];
      if (x_out) ((float4*)(x_out + t * d))[v] = a;
      if (save) ((float4*)(save + t * d))[v] = a;
      store4<T>(y + t * d + 4 * v, make_float4(gg.x * a.x * rr, gg.y * a.y * rr, gg.z * a.z * rr, gg.w * a.w * rr));
    }
  }
  if (threadIdx.x == 0) r[t] = rr;
}

template <typename T, int NVT, typename PT>
static void rms_fwd_launch(const float* x_in, const PT* parts, int nsplit, long ps, float* x_out, float* save,
                           const float* g, int n, int d, float eps, T* y, float* r, hipStream_t st) {
  hipLaunchKernelGGL((rms_fwd_kernel<T, NVT, PT>), dim3(n), dim3(RB), 0, st, x_in, parts, nsplit, ps, x_out, save, g,
                     d, eps, y, r);
}

template <typename T, typename PT>
static hipError_t rms_fwd_t(const float* x_in, const PT* parts, int nsplit, long ps, float* x_out, float* save,
                            const float* g, int n, int d, float eps, T* y, float* r, hipStream_t st) {
  const int nvt = (d / 4 + RB - 1) / RB;
  switch (nvt) {
    case 1: rms_fwd_launch<T, 1>(x_in, parts, nsplit, ps, x_out, save, g, n, d, eps, y, r, st); break;
    case 2: rms_fwd_launch<T, 2>(x_in, parts, nsplit, ps, x_out, save, g, n, d, eps, y, r, st); break;
    case 3: rms_fwd_launch<T, 3>(x_in, parts, nsplit, ps, x_out, save, g, n, d, eps, y, r, st); break;
    case 4: rms_fwd_launch<T, 4>(x_in, parts, nsplit, ps, x_out, save, g, n, d, eps, y, r, st); break;
    case 5:
    case 6: rms_fwd_launch<T, 6>(x_in, parts, nsplit, ps, x_out, save, g, n, d, eps, y, r, st); break;
    case 7:
    case 8: rms_fwd_launch<T, 8>(x_in, parts, nsplit, ps, x_out, save, g, n, d, eps, y, r, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t rmsnorm_fwd_fused(DT dt, const float* x_in, const float* parts, int nsplit, float* x_out, float* save,
                             const float* g, int n, int d, float eps, void* y, float* r, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (d % 4 || d > 4 * RB * RMS_MAXV) return hipErrorInvalidValue;
  const long ps = (long)n * d;
  if (dt == DT::BF16) return rms_fwd_t<bf16>(x_in, parts, nsplit, ps, x_out, save, g, n, d, eps, (bf16*)y, r, st);
  return rms_fwd_t<float>(x_in, parts, nsplit, ps, x_out, save, g, n, d, eps, (float*)y, r, st);
}

hipError_t rmsnorm_fwd_fused(DT dt, const float* x_in, const __bf16* parts, int nsplit, float* x_out, float* save,
                             const float* g, int n, int d, float eps, void* y, float* r, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (d % 4 || d > 4 * RB * RMS_MAXV) return hipErrorInvalidValue;
  const long ps = (long)n * d;
  if (dt == DT::BF16) return rms_fwd_t<bf16>(x_in, parts, nsplit, ps, x_out, save, g, n, d, eps, (bf16*)y, r, st);
  return rms_fwd_t<float>(x_in, parts, nsplit, ps, x_out, save, g, n, d, eps, (float*)y, r, st);
}

hipError_t rmsnorm_fwd(DT dt, const float* x, const float* g, int n, int d, float eps, void* y,
                       float* r, hipStream_t st) {
  return rmsnorm_fwd_fused(dt, x, (const float*)nullptr, 0, nullptr, nullptr, g, n, d, eps, y, r, st);
}

// dx = r (g dy) - x r^3 mean((g dy) x); dh (+)= dx; dh_t = T(dh); dy is the
// sum of nsplit partials. Every input of the row (the partials, g, x and,
// when accumulating, dh) is requested before the first use and kept in
// registers (NVT float4 chunks per thread, as in the forward).
template <typename T, int NVT, typename PT>
__global__ void __launch_bounds__(RB) rms_bwd_kernel(const PT* dy, int nsplit, long sstride, const float* x,
                                                     const float* g, const float* r, int d, float* dh, T* dh_t,
                                                     int acc) {
  __shared__ float sh[RB / 64];
  const long t = blockIdx.x;
  const float rr = r[t];
  const int nv = d / 4;
  float4 a[NVT], gv[NVT], xv[NVT], hv[NVT];
#pragma unroll
  for (int i = 0; i < NVT; ++i) {
    const int v = min((int)threadIdx.x + i * RB, nv - 1);
    a[i] = ld_part4(dy + t * d, v);
    gv[i] = ((const float4*)g)[v];
    xv[i] = ((const float4*)(x + t * d))[v];
  }
  if (acc) {  // uniform
#pragma unroll
    for (int i = 0; i < NVT; ++i) hv[i] = ((const float4*)(dh + t * d))[min((int)threadIdx.x + i * RB, nv - 1)];
  }
  rms_add_parts<NVT, PT>(a, dy + sstride, sstride, nsplit - 1, t * d, nv);
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < NVT; ++i)
    if (threadIdx.x + i * RB < nv) {
      const float4 gg = gv[i], xx = xv[i];
      a[i] = make_float4(a[i].x * gg.x, a[i].y * gg.y, a[i].z * gg.z, a[i].w * gg.w);  // g dy
      dot += a[i].x * xx.x + a[i].y * xx.y + a[i].z * xx.z + a[i].w * xx.w;
    }
  dot = block_sum(dot, sh) / d;
  const float c = rr * rr * rr * dot;
#pragma unroll
  for (int i = 0; i < NVT; ++i) {
    const int v = threadIdx.x + i * RB;
    if (v < nv) {
      const float4 q = a[i], xx = xv[i];
      float4 o = make_float4(rr * q.x - xx.x * c, rr * q.y - xx.y * c, rr * q.z - xx.z * c, rr * q.w - xx.w * c);
      if (acc) o = f4add(o, hv[i]);
      ((float4*)(dh + t * d))[v] = o;
      if (dh_t) store4<T>(dh_t + t * d + 4 * v, o);
    }
  }
}

template <typename T, int NVT, typename PT>
static void rms_bwd_launch(const PT* dy, int nsplit, long ss, const float* x, const float* g, const float* r,
                           int n, int d, float* dh, T* dh_t, int acc, hipStream_t st) {
  hipLaunchKernelGGL((rms_bwd_kernel<T, NVT, PT>), dim3(n), dim3(RB), 0, st, dy, nsplit, ss, x, g, r, d, dh, dh_t,
                     acc);
}

template <typename T, typename PT>
static hipError_t rms_bwd_t(const PT* dy, int nsplit, long ss, const float* x, const float* g, const float* r,
                            int n, int d, float* dh, T* dh_t, int acc, hipStream_t st) {
  const int nvt = (d / 4 + RB - 1) / RB;
  switch (nvt) {
    case 1: rms_bwd_launch<T, 1, PT>(dy, nsplit, ss, x, g, r, n, d, dh, dh_t, acc, st); break;
    case 2: rms_bwd_launch<T, 2, PT>(dy, nsplit, ss, x, g, r, n, d, dh, dh_t, acc, st); break;
    case 3: rms_bwd_launch<T, 3, PT>(dy, nsplit, ss, x, g, r, n, d, dh, dh_t, acc, st); break;
    case 4: rms_bwd_launch<T, 4, PT>(dy, nsplit, ss, x, g, r, n, d, dh, dh_t, acc, st); break;
    case 5:
    case 6: rms_bwd_launch<T, 6, PT>(dy, nsplit, ss, x, g, r, n, d, dh, dh_t, acc, st); break;
    case 7:
    case 8: rms_bwd_launch<T, 8, PT>(dy, nsplit, ss, x, g, r, n, d, dh, dh_t, acc, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t rmsnorm_bwd(DT dt, const void* dy, bool dy_bf16, int nsplit, const float* x, const float* g,
                       const float* r, int n, int d, float* dh, void* dh_t, int accumulate, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (d % 4 || nsplit < 1 || d > 4 * RB * RMS_MAXV) return hipErrorInvalidValue;
  const long ss = (long)n * d;
  if (dt == DT::BF16) {
    if (dy_bf16) return rms_bwd_t<bf16>((const bf16*)dy, nsplit, ss, x, g, r, n, d, dh, (bf16*)dh_t, accumulate, st);
    return rms_bwd_t<bf16>((const float*)dy, nsplit, ss, x, g, r, n, d, dh, (bf16*)dh_t, accumulate, st);
  }
  if (dy_bf16) return hipErrorInvalidValue;
  return rms_bwd_t<float>((const float*)dy, nsplit, ss, x, g, r, n, d, dh, (float*)dh_t, accumulate, st);
}

// -------------------------------------------------------------------- RoPE
// Half-split rotation: (x1, x2) -> (x1 c - x2 s, x1 s + x2 c), with (c, s)
// at tab[pos * dh/2 + j] (built on the host from float64 angles).
template <typename T>
__global__ void rope_scatter_generic_kernel(const T* qkv, int n, int H, int Hk, int dh, int64_t pos0,
                                    const float2* tab, T* q, T* ks, T* vs, int cap,
                                    int64_t min_pos) {
  const int t = blockIdx.x;
  const int64_t pos = pos0 + t;
  const int half = dh / 2;
  const int W = (H + 2 * Hk) * dh;
  const T* row = qkv + (long)t * W;
  const float2* tb = tab + pos * half;
  const bool store = pos >= min_pos;
  const long slot = (long)(pos & (cap - 1));
  // q and k heads: pairs
  for (int i = threadIdx.x; i < (H + Hk) * half; i += blockDim.x) {
    const int hh = i / half, j = i % half;
    const float2 cs = tb[j];
    const float x1 = to_f(row[hh * dh + j]), x2 = to_f(row[hh * dh + j + half]);
    const float y1 = x1 * cs.x - x2 * cs.y, y2 = x1 * cs.y + x2 * cs.x;
    if (hh < H) {
      q[((long)t * H + hh) * dh + j] = from_f<T>(y1);
      q[((long)t * H + hh) * dh + j + half] = from_f<T>(y2);
    } else if (store) {
      const int kh = hh - H;
      ks[((long)kh * cap + slot) * dh + j] = from_f<T>(y1);
      ks[((long)kh * cap + slot) * dh + j + half] = from_f<T>(y2);
    }
  }
  if (store)
    for (int i = threadIdx.x; i < Hk * dh; i += blockDim.x) {
      const int kh = i / dh, j = i % dh;
      vs[((long)kh * cap + slot) * dh + j] = row[(H + Hk) * dh + i];
    }
}

// Four consecutive elements of a row (T) as floats.
template <typename T> struct Vec4;
template <> struct Vec4<bf16> {
  typedef bf16x4 raw;
  __device__ __forceinline__ static float4 f(raw v) {
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
  }
};
template <> struct Vec4<float> {
  typedef float4 raw;
  __device__ __forceinline__ static float4 f(raw v) { return v; }
};

// One workgroup per token; thread i takes the rotation groups i, i + RB, ...
// (KR at most: 4 consecutive pairs (j .. j+3, j+dh/2 .. j+dh/2+3) of one q
// or k head) and the i-th 16-byte vector of the token's values. Every load
// is issued before the first store: the memory counter that tracks loads
// also tracks stores, so interleaving them would cost a round trip each.
// Shapes past its limits ((H + Hk) dh / 8 groups at most ROPE_KR * RB, Hk
// dh values at most RB 16-byte vectors) take the element-wise kernel above
// (rope_scatter chooses).
constexpr int ROPE_KR = 4;
template <typename T>
__global__ void __launch_bounds__(RB) rope_scatter_kernel(const T* qkv, int n, int H, int Hk, int dh, int64_t pos0,
                                                          const float2* tab, T* q, T* ks, T* vs, int cap,
                                                          int64_t min_pos) {
  typedef typename Vec4<T>::raw R4;
  constexpr int VE = 16 / sizeof(T);
  const int t = blockIdx.x;
  const int64_t pos = pos0 + t;
  const int half = dh / 2;
  const int W = (H + 2 * Hk) * dh;
  const T* row = qkv + (long)t * W;
  const float4* tb = (const float4*)(tab + pos * half);  // (c, s) of pairs j and j + 1
  const bool store = pos >= min_pos;
  const long slot = (long)(pos & (cap - 1));
  const int gph = half / 4, ng = (H + Hk) * gph, nvv = Hk * dh / VE;
  R4 x1[ROPE_KR], x2[ROPE_KR];
  float4 c01[ROPE_KR], c23[ROPE_KR];
  uint4 vv;
#pragma unroll
  for (int k = 0; k < ROPE_KR; ++k) {
    // unconditional loads from a clamped (valid) group: a load under the
    // lane condition becomes a branch with its own wait for memory
    const int gi = min((int)threadIdx.x + k * RB, ng - 1);
    const int hh = gi / gph, j = (gi % gph) * 4;
    x1[k] = *(const R4*)(row + hh * dh + j);
    x2[k] = *(const R4*)(row + hh * dh + j + half);
    c01[k] = tb[j / 2];
    c23[k] = tb[j / 2 + 1];
  }
  const bool hv = store && (int)threadIdx.x < nvv;
  vv = ((const uint4*)(row + (H + Hk) * dh))[min((int)threadIdx.x, nvv - 1)];
#pragma unroll
  for (int k = 0; k < ROPE_KR; ++k) {
    const int gi = threadIdx.x + k * RB;
    if (gi >= ng) continue;
    const int hh = gi / gph, j = (gi % gph) * 4;
    T* d;
    if (hh < H) d = q + ((long)t * H + hh) * dh + j;
    else if (store) d = ks + ((long)(hh - H) * cap + slot) * dh + j;
    else continue;
    const float4 a = Vec4<T>::f(x1[k]), b = Vec4<T>::f(x2[k]);
    const float4 c = c01[k], e = c23[k];
    store4<T>(d, make_float4(a.x * c.x - b.x * c.y, a.y * c.z - b.y * c.w, a.z * e.x - b.z * e.y,
                             a.w * e.z - b.w * e.w));
    store4<T>(d + half, make_float4(a.x * c.y + b.x * c.x, a.y * c.w + b.y * c.z, a.z * e.y + b.z * e.x,
                                    a.w * e.w + b.w * e.z));
  }
  if (hv) {
    const int e0 = threadIdx.x * VE, kh = e0 / dh, j = e0 % dh;
    *(uint4*)(vs + ((long)kh * cap + slot) * dh + j) = vv;
  }
}

// The transposed value store: a workgroup takes 64 tokens of one key head
// and DS of its dh rows (blockIdx.z selects which), loads their values as
// 16-byte vectors (all loads issued before the first LDS write), stages them
// in LDS and writes each row of the store as 64 consecutive positions
// (vt_slot permutes within aligned groups of 16, so a wave's stores still
// cover whole 128-byte runs).
template <typename T>
__global__ void __launch_bounds__(256) vt_scatter_kernel(const T* qkv, int n, int H, int Hk, int dh, int64_t pos0,
                                                         T* vts, int cap, int64_t min_pos) {
  extern __shared__ unsigned char vt_lds[];
  T* Vs = (T*)vt_lds;  // [ds][65]
  constexpr int TT = 64, PITCH = TT + 1;
  constexpr int VE = 16 / sizeof(T);
  const int t0 = blockIdx.x * TT, kh = blockIdx.y;
  const int ds = dh / gridDim.z, d0 = blockIdx.z * ds;
  const int W = (H + 2 * Hk) * dh;
  const int vpr = ds / VE;  // 16-byte vectors per token row
  constexpr int MAXL = 4;   // vectors per thread (TT * ds / VE <= 256 * MAXL)
  uint4 r[MAXL];
#pragma unroll
  for (int i = 0; i < MAXL; ++i) {
    // unconditional loads from a clamped (valid) token row (a load under the
    // lane condition becomes a branch with its own wait for memory)
    const int e = threadIdx.x + i * 256, t = min(e / vpr, TT - 1), v = e % vpr;
    r[i] = *(const uint4*)(qkv + (long)min(t0 + t, n - 1) * W + (H + Hk) * dh + kh * dh + d0 + v * VE);
  }
#pragma unroll
  for (int i = 0; i < MAXL; ++i) {
    const int e = threadIdx.x + i * 256, t = e / vpr, v = e % vpr;
    if (t < TT && t0 + t < n) {
      const T* x = (const T*)&r[i];
#pragma unroll
      for (int k = 0; k < VE; ++k) Vs[(v * VE + k) * PITCH + t] = x[k];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < TT * ds; e += blockDim.x) {
    const int d = e / TT, t = e % TT;
    const int64_t pos = pos0 + t0 + t;
    if (t0 + t < n && pos >= min_pos)
      vts[((long)kh * dh + d0 + d) * cap + vt_slot(pos & (cap - 1))] = Vs[d * PITCH + t];
  }
}

hipError_t rope_scatter(DT dt, const void* qkv, int n, int H, int Hk, int dh, int64_t pos0,
                        const float2* tab, void* q, void* ks, void* vs, void* vts, int cap,
                        int64_t min_pos, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  // dh split in two for dh 128 (more workgroups for a mini-batch); each
  // part must be whole 16-byte vectors and fit the loader (64 x part <= 256 x 4 vectors)
  const int esz = (int)dt_size(dt);
  int dsp = (dh >= 128) ? 2 : 1;
  while (dsp > 1 && ((dh / dsp) * esz) % 16) dsp = 1;
  if (((dh / dsp) * esz) % 16 || 64 * (dh / dsp) * esz / 16 > 256 * 4) return hipErrorInvalidValue;
  const dim3 vgrid((n + 63) / 64, Hk, dsp);
  const size_t vlds = (size_t)(dh / dsp) * 65;
  // the vector kernel: whole 4-pair groups, at most ROPE_KR per thread, and
  // one 16-byte value vector per thread
  const bool vec = dh % 8 == 0 && (H + Hk) * (dh / 8) <= ROPE_KR * RB && Hk * dh * esz / 16 <= RB &&
                   (dh * esz) % 16 == 0;
  if (dt == DT::BF16) {
    if (vec)
      hipLaunchKernelGGL(rope_scatter_kernel<bf16>, dim3(n), dim3(RB), 0, st, (const bf16*)qkv, n, H, Hk,
                         dh, pos0, tab, (bf16*)q, (bf16*)ks, (bf16*)vs, cap, min_pos);
    else
      hipLaunchKernelGGL(rope_scatter_generic_kernel<bf16>, dim3(n), dim3(RB), 0, st, (const bf16*)qkv, n, H, Hk,
                         dh, pos0, tab, (bf16*)q, (bf16*)ks, (bf16*)vs, cap, min_pos);
    if (vts)
      hipLaunchKernelGGL(vt_scatter_kernel<bf16>, vgrid, dim3(256), vlds * sizeof(bf16), st,
                         (const bf16*)qkv, n, H, Hk, dh, pos0, (bf16*)vts, cap, min_pos);
  } else {
    if (vec)
      hipLaunchKernelGGL(rope_scatter_kernel<float>, dim3(n), dim3(RB), 0, st, (const float*)qkv, n, H,
                         Hk, dh, pos0, tab, (float*)q, (float*)ks, (float*)vs, cap, min_pos);
    else
      hipLaunchKernelGGL(rope_scatter_generic_kernel<float>, dim3(n), dim3(RB), 0, st, (const float*)qkv, n, H,
                         Hk, dh, pos0, tab, (float*)q, (float*)ks, (float*)vs, cap, min_pos);
    if (vts)
      hipLaunchKernelGGL(vt_scatter_kernel<float>, vgrid, dim3(256), vlds * sizeof(float), st,
                         (const float*)qkv, n, H, Hk, dh, pos0, (float*)vts, cap, min_pos);
  }
  return hipGetLastError();
}

// Transpose of the rotation (rotation by -angle) for dq, dk; dv copied.
// Partial sums of dk, dv at position t: kv_parts, or with kv_run > 0 those
// of t's key block in the dK / dV kernel's runs.
__device__ __forceinline__ int rope_kv_parts(int kv_parts, int kv_run, int kv_window, int n, int H, int Hk, int t) {
  return kv_run > 0 ? attn_bwd2_kv_block_parts(n, kv_window, H / Hk, kv_run, t >> 7) : kv_parts;
}

template <typename T, typename PT>
__global__ void rope_bwd_generic_kernel(const PT* dq, int dq_parts, const PT* dk, const PT* dv, int kv_parts_all,
                                        int kv_run, int kv_window, int n, int H, int Hk, int dh, int64_t pos0,
                                        const float2* tab, T* out) {
  const int t = blockIdx.x;
  const int kv_parts = rope_kv_parts(kv_parts_all, kv_run, kv_window, n, H, Hk, t);
  const int half = dh / 2;
  const int W = (H + 2 * Hk) * dh;
  const long qstride = (long)n * H * dh, kstride = (long)n * Hk * dh;
  const float2* tb = tab + (pos0 + t) * half;
  // partial sums (query-side key splits, per-query-head key gradients) are
  // added in a fixed order
  for (int i = threadIdx.x; i < (H + Hk) * half; i += blockDim.x) {
    const int hh = i / half, j = i % half;
    const float2 cs = tb[j];
    const bool isq = hh < H;
    const PT* src = isq ? dq + ((long)t * H + hh) * dh : dk + ((long)t * Hk + (hh - H)) * dh;
    const int np = isq ? dq_parts : kv_parts;
    const long ps = isq ? qstride : kstride;
    float g1 = 0.f, g2 = 0.f;
    for (int p = 0; p < np; ++p) {
      g1 += to_f(src[p * ps + j]);
      g2 += to_f(src[p * ps + j + half]);
    }
    out[(long)t * W + hh * dh + j] = from_f<T>(g1 * cs.x + g2 * cs.y);
    out[(long)t * W + hh * dh + j + half] = from_f<T>(-g1 * cs.y + g2 * cs.x);
  }
  for (int i = threadIdx.x; i < Hk * dh; i += blockDim.x) {
    float g = 0.f;
    for (int p = 0; p < kv_parts; ++p) g += to_f(dv[p * kstride + (long)t * Hk * dh + i]);
    out[(long)t * W + (H + Hk) * dh + i] = from_f<T>(g);
  }
}

// The same, vectorized: thread i takes rotation groups i and i + RB (4
// consecutive pairs of one head; ROPE_BKR at most) and the i-th group of 4
// value-gradient elements; the loads of every partial are issued before the
// first store. At most ROPE_BNP partials per side (rope_bwd_pack chooses).
constexpr int ROPE_BKR = 2, ROPE_BNP = 8;
template <typename T, typename PT>
__global__ void __launch_bounds__(RB) rope_bwd_kernel(const PT* dq, int dq_parts, const PT* dk, const PT* dv,
                                                      int kv_parts_all, int kv_run, int kv_window, int n, int H,
                                                      int Hk, int dh, int64_t pos0, const float2* tab, T* out) {
  const int t = blockIdx.x;
  const int kv_parts = rope_kv_parts(kv_parts_all, kv_run, kv_window, n, H, Hk, t);
  const int half = dh / 2;
  const int W = (H + 2 * Hk) * dh;
  const long qstride = (long)n * H * dh, kstride = (long)n * Hk * dh;
  const float4* tb = (const float4*)(tab + (pos0 + t) * half);
  const int gph = half / 4, ng = (H + Hk) * gph, nvg = Hk * dh / 4;
  float4 g1[ROPE_BKR][ROPE_BNP], g2[ROPE_BKR][ROPE_BNP], c01[ROPE_BKR], c23[ROPE_BKR], gv[ROPE_BNP];
#pragma unroll
  for (int k = 0; k < ROPE_BKR; ++k) {
    const int gi = threadIdx.x + k * RB;
    if (gi < ng) {
      const int hh = gi / gph, j = (gi % gph) * 4;
      const bool isq = hh < H;
      const PT* src = isq ? dq + ((long)t * H + hh) * dh : dk + ((long)t * Hk + (hh - H)) * dh;
      const int np = isq ? dq_parts : kv_parts;
      const long ps = isq ? qstride : kstride;
#pragma unroll
      for (int p = 0; p < ROPE_BNP; ++p)
        if (p < np) {
          g1[k][p] = ld_part4(src + p * ps + j, 0);
          g2[k][p] = ld_part4(src + p * ps + j + half, 0);
        }
      c01[k] = tb[j / 2];
      c23[k] = tb[j / 2 + 1];
    }
  }
  const bool hv = (int)threadIdx.x < nvg;
#pragma unroll
  for (int p = 0; p < ROPE_BNP; ++p)
    if (hv && p < kv_parts) gv[p] = ld_part4(dv + p * kstride + (long)t * Hk * dh, threadIdx.x);
  // partial sums added in a fixed order
#pragma unroll
  for (int k = 0; k < ROPE_BKR; ++k) {
    const int gi = threadIdx.x + k * RB;
    if (gi >= ng) continue;
    const int hh = gi / gph, j = (gi % gph) * 4;
    const int np = hh < H ? dq_parts : kv_parts;
    float4 a = g1[k][0], b = g2[k][0];
#pragma unroll
    for (int p = 1; p < ROPE_BNP; ++p)
      if (p < np) {
        a = f4add(a, g1[k][p]);
        b = f4add(b, g2[k][p]);
      }
    const float4 c = c01[k], e = c23[k];
    T* d = out + (long)t * W + hh * dh + j;
    store4<T>(d, make_float4(a.x * c.x + b.x * c.y, a.y * c.z + b.y * c.w, a.z * e.x + b.z * e.y,
                             a.w * e.z + b.w * e.w));
    store4<T>(d + half, make_float4(-a.x * c.y + b.x * c.x, -a.y * c.w + b.y * c.z, -a.z * e.y + b.z * e.x,
                                    -a.w * e.w + b.w * e.z));
  }
  if (hv) {
    float4 g = gv[0];
#pragma unroll
    for (int p = 1; p < ROPE_BNP; ++p)
      if (p < kv_parts) g = f4add(g, gv[p]);
    store4<T>(out + (long)t * W + (H + Hk) * dh + 4 * threadIdx.x, g);
  }
}

template <typename PT>
static hipError_t rope_bwd_pack_t(DT dt, const PT* dq, int dq_parts, const PT* dk, const PT* dv, int kv_parts,
                                  int kv_run, int kv_window, int n, int H, int Hk, int dh, int64_t pos0,
                                  const float2* tab, void* dqkv, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const bool vec = dh % 8 == 0 && (H + Hk) * (dh / 8) <= ROPE_BKR * RB && Hk * dh / 4 <= RB && dq_parts >= 1 &&
                   dq_parts <= ROPE_BNP && kv_parts >= 1 && kv_parts <= ROPE_BNP;
  if (dt == DT::BF16) {
    if (vec)
      hipLaunchKernelGGL((rope_bwd_kernel<bf16, PT>), dim3(n), dim3(RB), 0, st, dq, dq_parts, dk, dv, kv_parts, kv_run, kv_window, n,
                         H, Hk, dh, pos0, tab, (bf16*)dqkv);
    else
      hipLaunchKernelGGL((rope_bwd_generic_kernel<bf16, PT>), dim3(n), dim3(RB), 0, st, dq, dq_parts, dk, dv, kv_parts, kv_run,
                         kv_window, n, H, Hk, dh, pos0, tab, (bf16*)dqkv);
  } else {
    if (vec)
      hipLaunchKernelGGL((rope_bwd_kernel<float, PT>), dim3(n), dim3(RB), 0, st, dq, dq_parts, dk, dv, kv_parts, kv_run, kv_window, n,
                         H, Hk, dh, pos0, tab, (float*)dqkv);
    else
      hipLaunchKernelGGL((rope_bwd_generic_kernel<float, PT>), dim3(n), dim3(RB), 0, st, dq, dq_parts, dk, dv, kv_parts,
                         kv_run, kv_window, n, H, Hk, dh, pos0, tab, (float*)dqkv);
  }
  return hipGetLastError();
}

hipError_t rope_bwd_pack(DT dt, const float* dq, int dq_parts, const float* dk, const float* dv, int kv_parts,
                         int kv_run, int kv_window, int n, int H, int Hk, int dh, int64_t pos0, const float2* tab,
                         void* dqkv, hipStream_t st) {
  return rope_bwd_pack_t(dt, dq, dq_parts, dk, dv, kv_parts, kv_run, kv_window, n, H, Hk, dh, pos0, tab, dqkv, st);
}

hipError_t rope_bwd_pack(DT dt, const bf16* dq, int dq_parts, const bf16* dk, const bf16* dv, int kv_parts,
                         int kv_run, int kv_window, int n, int H, int Hk, int dh, int64_t pos0, const float2* tab,
                         void* dqkv, hipStream_t st) {
  return rope_bwd_pack_t(dt, dq, dq_parts, dk, dv, kv_parts, kv_run, kv_window, n, H, Hk, dh, pos0, tab, dqkv, st);
}

__global__ void sum_parts_kernel(const float* parts, int nparts, long count, float* dst) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < count; i += (long)gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int p = 0; p < nparts; ++p) s += parts[p * count + i];
    dst[i] = s;
  }
}

hipError_t sum_parts_f32(const float* parts, int nparts, long count, float* dst, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  const long blocks = std::min((count + 255) / 256, 4096L);
  hipLaunchKernelGGL(sum_parts_kernel, dim3((unsigned)blocks), dim3(256), 0, st, parts, nparts, count, dst);
  return hipGetLastError();
}

// ------------------------------------------------------- softmax CE + dz
// One workgroup per row: pass 1 keeps a per-thread running (max, sum-exp)
// over float4 chunks, combined across the block; pass 2 writes
// dz = (exp(z - lse) - [v == label]) * scale.
template <typename T>
__global__ void __launch_bounds__(RB) ce_kernel(const float* z, int nt, int V, const int32_t* lab,
                                                float scale, float* loss, T* dz, int* err) {
  __shared__ float shm[RB / 64], shs[RB / 64];
  const long t = blockIdx.x;
  const float* zr = z + t * V;
  T* dr = dz + t * V;
  if ((int)t >= nt) {
    for (int j = threadIdx.x; j < V; j += blockDim.x) dr[j] = from_f<T>(0.f);
    return;
  }
  float m = -INFINITY, s = 0.f;
  const float4* z4 = (const float4*)zr;
  const int nv4 = V / 4;
  // four float4 chunks per thread per round, loaded before they are used
  constexpr int U = 4;
  int j = threadIdx.x;
  for (; j + (U - 1) * RB < nv4; j += U * RB) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = z4[j + u * RB];
    float mx = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mx = fmaxf(mx, fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)));
    if (mx == -INFINITY) continue;  // nothing finite yet (s is still 0)
    s *= __expf(m - mx);
    m = mx;
#pragma unroll
    for (int u = 0; u < U; ++u)
      s += __expf(v[u].x - m) + __expf(v[u].y - m) + __expf(v[u].z - m) + __expf(v[u].w - m);
  }
  for (; j < nv4; j += RB) {
    const float4 v = z4[j];
    const float mx = fmaxf(m, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
    if (mx == -INFINITY) continue;
    s *= __expf(m - mx);
    m = mx;
    s += __expf(v.x - m) + __expf(v.y - m) + __expf(v.z - m) + __expf(v.w - m);
  }
  // combine (m, s) across the wave, then the block
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    const float mn = fmaxf(m, m2);
    s = (m == -INFINITY ? 0.f : s * __expf(m - mn)) + (m2 == -INFINITY ? 0.f : s2 * __expf(m2 - mn));
    m = mn;
  }
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) {
    shm[w] = m;
    shs[w] = s;
  }
  __syncthreads();
  float M = -INFINITY;
  for (int i = 0; i < RB / 64; ++i) M = fmaxf(M, shm[i]);
  float S = 0.f;
  for (int i = 0; i < RB / 64; ++i) S += shs[i] * __expf(shm[i] - M);
  const float lse = M + __logf(S);
  const int y = lab[t];
  const bool yok = y >= 0 && y < V;
  if (threadIdx.x == 0) {
    const float li = yok ? lse - zr[y] : NAN;
    loss[t] = li;
    if (!yok) atomicOr(err, 1);
    else if (!isfinite(li)) atomicOr(err, 4);
  }
  auto dz4 = [&](float4 v, int b) {
    return make_float4((__expf(v.x - lse) - (b + 0 == y ? 1.f : 0.f)) * scale,
                       (__expf(v.y - lse) - (b + 1 == y ? 1.f : 0.f)) * scale,
                       (__expf(v.z - lse) - (b + 2 == y ? 1.f : 0.f)) * scale,
                       (__expf(v.w - lse) - (b + 3 == y ? 1.f : 0.f)) * scale);
  };
  j = threadIdx.x;
  for (; j + (U - 1) * RB < nv4; j += U * RB) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = z4[j + u * RB];
#pragma unroll
    for (int u = 0; u < U; ++u) store4<T>(dr + 4 * (j + u * RB), dz4(v[u], 4 * (j + u * RB)));
  }
  for (; j < nv4; j += RB) store4<T>(dr + 4 * j, dz4(z4[j], 4 * j));
}

hipError_t ce_fwd_bwd(DT dt, const float* z, int n, int nt, int V, const int32_t* lab, float scale,
                      float* loss, void* dz, int* err, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (V % 4) return hipErrorInvalidValue;
  if (dt == DT::BF16)
    hipLaunchKernelGGL(ce_kernel<bf16>, dim3(n), dim3(RB), 0, st, z, nt, V, lab, scale, loss, (bf16*)dz, err);
  else
    hipLaunchKernelGGL(ce_kernel<float>, dim3(n), dim3(RB), 0, st, z, nt, V, lab, scale, loss, (float*)dz,
                       err);
  return hipGetLastError();
}

// Softmax CE + logit gradient from per-64-column (max, sum exp) partials of
// the logits (written by the lm_head product's epilogue): the row's
// log-sum-exp comes from its ceil(V / 64) partials, so the logits are read
// once, for dz = (exp(z - lse) - [v == label]) * scale and the label's
// logit. One workgroup per row.
template <typename T>
__global__ void __launch_bounds__(RB) ce_lse_kernel(const float* z, const float2* parts, int nt, int V,
                                                    const int32_t* lab, float scale, float* loss, T* dz,
                                                    int* err) {
  __shared__ float shm[RB / 64], shs[RB / 64];
  const long t = blockIdx.x;
  const float* zr = z + t * V;
  T* dr = dz + t * V;
  if ((int)t >= nt) {
    for (int j = threadIdx.x; j < V; j += blockDim.x) dr[j] = from_f<T>(0.f);
    return;
  }
  const int np = (V + 63) / 64;
  const float2* pr = parts + t * np;
  float m = -INFINITY, s = 0.f;
  for (int j = threadIdx.x; j < np; j += RB) {
    const float2 p = pr[j];
    if (p.x == -INFINITY) continue;
    const float mn = fmaxf(m, p.x);
    s = (m == -INFINITY ? 0.f : s * __expf(m - mn)) + p.y * __expf(p.x - mn);
    m = mn;
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    const float mn = fmaxf(m, m2);
    s = (m == -INFINITY ? 0.f : s * __expf(m - mn)) + (m2 == -INFINITY ? 0.f : s2 * __expf(m2 - mn));
    m = mn;
  }
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) {
    shm[w] = m;
    shs[w] = s;
  }
  __syncthreads();
  float M = -INFINITY;
  for (int i = 0; i < RB / 64; ++i) M = fmaxf(M, shm[i]);
  float S = 0.f;
  for (int i = 0; i < RB / 64; ++i) S += shm[i] == -INFINITY ? 0.f : shs[i] * __expf(shm[i] - M);
  const float lse = M + __logf(S);
  const int y = lab[t];
  const bool yok = y >= 0 && y < V;
  if (threadIdx.x == 0) {
    const float li = yok ? lse - zr[y] : NAN;
    loss[t] = li;
    if (!yok) atomicOr(err, 1);
    else if (!isfinite(li)) atomicOr(err, 4);
  }
  auto dz4 = [&](float4 v, int b) {
    return make_float4((__expf(v.x - lse) - (b + 0 == y ? 1.f : 0.f)) * scale,
                       (__expf(v.y - lse) - (b + 1 == y ? 1.f : 0.f)) * scale,
                       (__expf(v.z - lse) - (b + 2 == y ? 1.f : 0.f)) * scale,
                       (__expf(v.w - lse) - (b + 3 == y ? 1.f : 0.f)) * scale);
  };
  const float4* z4 = (const float4*)zr;
  const int nv4 = V / 4;
  constexpr int U = 4;
  int j = threadIdx.x;
  for (; j + (U - 1) * RB < nv4; j += U * RB) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = z4[j + u * RB];
#pragma unroll
    for (int u = 0; u < U; ++u) store4<T>(dr + 4 * (j + u * RB), dz4(v[u], 4 * (j + u * RB)));
  }
  for (; j < nv4; j += RB) store4<T>(dr + 4 * j, dz4(z4[j], 4 * j));
}

hipError_t ce_fwd_bwd_lse(DT dt, const float* z, const float2* parts, int n, int nt, int V, const int32_t* lab,
                          float scale, float* loss, void* dz, int* err, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (dt != DT::BF16 || V % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ce_lse_kernel<bf16>, dim3(n), dim3(RB), 0, st, z, parts, nt, V, lab, scale, loss, (bf16*)dz,
                     err);
  return hipGetLastError();
}

// ------------------------------------------------------------ rowdot D
// D[h][t] = dO[t, h, :] . O[t, h, :]. A row (t, h) is dh * sizeof(T) bytes,
// taken by LPR lanes reading 16 bytes each from both operands (every load of
// a lane issued before the products), the LPR partial sums meeting through
// lane shuffles; a 64-lane wave covers 64 / LPR rows.
template <typename T, int LPR>
__global__ void __launch_bounds__(256) rowdot_kernel(const T* dO, const T* O, int n, int H, int dh, float* D) {
  constexpr int VE = 16 / sizeof(T);
  const long rows = (long)n * H;
  const long w = ((long)blockIdx.x * 256 + threadIdx.x) / LPR;  // row of this lane
  const int sub = threadIdx.x % LPR;
  const int nvr = dh / VE;  // 16-byte vectors per row
  float s = 0.f;
  if (w < rows) {
    constexpr int MAXV = 4;  // vectors per lane (dh * sizeof(T) <= 64 LPR bytes)
    uint4 a[MAXV], c[MAXV];
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int v = sub + i * LPR;
      if (v < nvr) {
        a[i] = ((const uint4*)(dO + w * dh))[v];
        c[i] = ((const uint4*)(O + w * dh))[v];
      }
    }
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      if (sub + i * LPR >= nvr) continue;
      const T* x = (const T*)&a[i];
      const T* y = (const T*)&c[i];
#pragma unroll
      for (int e = 0; e < VE; ++e) s += to_f(x[e]) * to_f(y[e]);
    }
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (w < rows && sub == 0) {
    const long t = w / H, h = w % H;
    D[h * n + t] = s;
  }
}

hipError_t attn_rowdot(DT dt, const void* dO, const void* O, int n, int H, int dh, float* D,
                       hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const long rows = (long)n * H;
  const int es = (int)dt_size(dt);
  if ((dh * es) % 16 || dh * es > 16 * 16 * 4) return hipErrorInvalidValue;
  // lanes per row: 16 for rows of up to 256 bytes, else 16 with several vectors each
  constexpr int LPR = 16;
  const dim3 grid((unsigned)((rows * LPR + 255) / 256));
  if (dt == DT::BF16)
    hipLaunchKernelGGL((rowdot_kernel<bf16, LPR>), grid, dim3(256), 0, st, (const bf16*)dO, (const bf16*)O, n, H, dh, D);
  else
    hipLaunchKernelGGL((rowdot_kernel<float, LPR>), grid, dim3(256), 0, st, (const float*)dO, (const float*)O, n, H,
                       dh, D);
  return hipGetLastError();
}

// ------------------------------------------------------------- helpers
__global__ void copy_f32_kernel(const float* s, float* d, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    d[i] = s[i];
}
template <typename T>
__global__ void cast_to_kernel(const float* s, T* d, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    d[i] = from_f<T>(s[i]);
}
template <typename T>
__global__ void cast_from_kernel(const T* s, float* d, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    d[i] = to_f(s[i]);
}
__global__ void fill_i32_kernel(int* p, int v, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}
__global__ void fill_f32_kernel(float* p, float v, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}
__global__ void fill_u32_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}
__global__ void fill_u8_kernel(uint8_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

static dim3 grid_for(size_t n) {
  size_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  if (b == 0) b = 1;
  return dim3((unsigned)b);
}

hipError_t copy_f32(const float* s, float* d, size_t n, hipStream_t st) {
  if (!n) return hipSuccess;
  hipLaunchKernelGGL(copy_f32_kernel, grid_for(n), dim3(256), 0, st, s, d, n);
  return hipGetLastError();
}
hipError_t cast_to(DT dt, const float* s, void* d, size_t n, hipStream_t st) {
  if (!n) return hipSuccess;
  if (dt == DT::BF16) hipLaunchKernelGGL(cast_to_kernel<bf16>, grid_for(n), dim3(256), 0, st, s, (bf16*)d, n);
  else hipLaunchKernelGGL(cast_to_kernel<float>, grid_for(n), dim3(256), 0, st, s, (float*)d, n);
  return hipGetLastError();
}
hipError_t cast_from(DT dt, const void* s, float* d, size_t n, hipStream_t st) {
  if (!n) return hipSuccess;
  if (dt == DT::BF16)
    hipLaunchKernelGGL(cast_from_kernel<bf16>, grid_for(n), dim3(256), 0, st, (const bf16*)s, d, n);
  else hipLaunchKernelGGL(cast_from_kernel<float>, grid_for(n), dim3(256), 0, st, (const float*)s, d, n);
  return hipGetLastError();
}
hipError_t fill_i32(int* p, int v, size_t n, hipStream_t st) {
  if (!n) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, grid_for(n), dim3(256), 0, st, p, v, n);
  return hipGetLastError();
}
hipError_t fill_f32(float* p, float v, size_t n, hipStream_t st) {
  if (!n) return hipSuccess;
  hipLaunchKernelGGL(fill_f32_kernel, grid_for(n), dim3(256), 0, st, p, v, n);
  return hipGetLastError();
}
hipError_t fill_zero_bytes(void* p, size_t nb, hipStream_t st) {
  if (!nb) return hipSuccess;
  if ((nb & 3) == 0 && ((uintptr_t)p & 3) == 0)
    hipLaunchKernelGGL(fill_u32_kernel, grid_for(nb / 4), dim3(256), 0, st, (uint32_t*)p, nb / 4);
  else
    hipLaunchKernelGGL(fill_u8_kernel, grid_for(nb), dim3(256), 0, st, (uint8_t*)p, nb);
  return hipGetLastError();
}

}  // namespace ttt
