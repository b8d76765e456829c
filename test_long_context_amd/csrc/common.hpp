// Shared device-side definitions for the TTT-E2E gfx950 kernels.
//
// Storage types: bf16 (clang's __bf16) for the bf16 workloads, float for the
// fp32 workload. All arithmetic accumulates in fp32. Matrix products use the
// CDNA4 MFMA units:
//   * bf16: v_mfma_f32_16x16x32_bf16 -- each lane supplies 8 consecutive K
//     elements of one row (A) / one column (B);
//   * fp32: v_mfma_f32_16x16x4_f32, issued 8 times with the same 8-per-lane
//     K grouping (instruction j consumes K = 8 g + j from lane group g), so
//     fragments have one shape for both storage types.
// The 16x16 fp32 accumulator holds, in lane l, rows 4 (l / 16) + r (r < 4) of
// column l % 16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

static constexpr int WAVE = 64;

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// 8 elements of T along the contraction dimension, one per lane slot.
template <typename T> struct Frag8;
template <> struct Frag8<bf16> { bf16x8 v; };
template <> struct Frag8<float> { floatx4 lo, hi; };

__device__ __forceinline__ void mma16(floatx4& acc, const Frag8<bf16>& a, const Frag8<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(floatx4& acc, const Frag8<float>& a, const Frag8<float>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], acc, 0, 0, 0);
}

// Load 8 consecutive elements (16-byte aligned for bf16, 32 for f32).
__device__ __forceinline__ void ld8(Frag8<bf16>& f, const bf16* p) { f.v = *(const bf16x8*)p; }
__device__ __forceinline__ void ld8(Frag8<float>& f, const float* p) {
  f.lo = *(const floatx4*)p;
  f.hi = *(const floatx4*)(p + 4);
}
__device__ __forceinline__ void st8(bf16* p, const Frag8<bf16>& f) { *(bf16x8*)p = f.v; }
__device__ __forceinline__ void st8(float* p, const Frag8<float>& f) {
  *(floatx4*)p = f.lo;
  *(floatx4*)(p + 4) = f.hi;
}
__device__ __forceinline__ void zero8(Frag8<bf16>& f) {
  for (int i = 0; i < 8; ++i) f.v[i] = (bf16)0.0f;
}
__device__ __forceinline__ void zero8(Frag8<float>& f) {
  f.lo = floatx4{0, 0, 0, 0};
  f.hi = floatx4{0, 0, 0, 0};
}
__device__ __forceinline__ float get8(const Frag8<bf16>& f, int i) { return (float)f.v[i]; }
__device__ __forceinline__ float get8(const Frag8<float>& f, int i) { return i < 4 ? f.lo[i] : f.hi[i - 4]; }
__device__ __forceinline__ void set8(Frag8<bf16>& f, int i, float x) { f.v[i] = (bf16)x; }
__device__ __forceinline__ void set8(Frag8<float>& f, int i, float x) {
  if (i < 4) f.lo[i] = x; else f.hi[i - 4] = x;
}

// Element access on raw Frag8 storage when the element is already of type T.
template <typename T> __device__ __forceinline__ T eget(const Frag8<T>& f, int i);
template <> __device__ __forceinline__ bf16 eget<bf16>(const Frag8<bf16>& f, int i) { return f.v[i]; }
template <> __device__ __forceinline__ float eget<float>(const Frag8<float>& f, int i) {
  return i < 4 ? f.lo[i] : f.hi[i - 4];
}
template <typename T> __device__ __forceinline__ void eset(Frag8<T>& f, int i, T x);
template <> __device__ __forceinline__ void eset<bf16>(Frag8<bf16>& f, int i, bf16 x) { f.v[i] = x; }
template <> __device__ __forceinline__ void eset<float>(Frag8<float>& f, int i, float x) {
  if (i < 4) f.lo[i] = x; else f.hi[i - 4] = x;
}

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }
__device__ __forceinline__ float sigm_f(float a) { return 1.0f / (1.0f + __expf(-a)); }

// Wave-wide reductions (64 lanes).
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace ttt

namespace ttt {
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));

// v_mfma_f32_32x32x16_bf16: lane l supplies row (A) / column (B) l % 32 and
// contraction elements 8 (l / 32) .. + 7; accumulator element j of lane l is
// row 8 (j / 4) + 4 (l / 32) + j % 4, column l % 32.
__device__ __forceinline__ void mma32(floatx16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
}  // namespace ttt
