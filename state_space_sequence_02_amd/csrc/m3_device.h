// m3_device.h -- device-side helpers shared by the gfx950 kernels.
#pragma once

#include "m3_internal.h"

namespace m3 {

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16 v) { return static_cast<float>(v); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return static_cast<bf16>(v); }

// Eight consecutive elements of an input row, widened to fp32.  One 16-byte load
// for bf16, two for fp32.  `p` must be aligned to 8 elements.
__device__ __forceinline__ void load8(const bf16* p, float (&v)[8]) {
  const uint4 raw = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Streaming (non-temporal) 16-byte global load/store, for data touched once.
__device__ __forceinline__ float4 ld_stream4(const float* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_stream4(float* p, float4 v) {
  const f32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(p));
}

// ---------------------------------------------------------------------------
// MFMA fragments.  A fragment is the 8 values one lane contributes to a
// 16x16 output tile over a 32-wide slice of the contraction:
//   A operand: row m = lane % 16, contraction slots 8*(lane/16) + 0..7
//   B operand: column n = lane % 16, the same contraction slots
// bf16: one v_mfma_f32_16x16x32_bf16.  fp32: eight v_mfma_f32_16x16x4_f32, slot j
// of every lane group in step j.  Any assignment of contraction indices to slots
// is valid as long as the A and B fragments of one product use the same one.
// Output tile (both): lane holds D[4*(lane/16) + i][lane % 16], i = 0..3.
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ void frag_set(Frag<bf16>& f, int j, float x) { f.v[j] = static_cast<bf16>(x); }
__device__ __forceinline__ void frag_set(Frag<float>& f, int j, float x) { f.v[j] = x; }
__device__ __forceinline__ float frag_get(const Frag<bf16>& f, int j) { return static_cast<float>(f.v[j]); }
__device__ __forceinline__ float frag_get(const Frag<float>& f, int j) { return f.v[j]; }

template <typename T> __device__ __forceinline__ void frag_zero(Frag<T>& f) {
#pragma unroll
  for (int j = 0; j < 8; ++j) frag_set(f, j, 0.f);
}

// Loads 8 contiguous elements of type T from LDS into a fragment.
__device__ __forceinline__ void frag_lds8(Frag<bf16>& f, const bf16* p) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void frag_lds8(Frag<float>& f, const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
// Loads two runs of 4 contiguous elements (slots 0..3 and 4..7).
__device__ __forceinline__ void frag_lds4x2(Frag<bf16>& f, const bf16* p0, const bf16* p1) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void frag_lds4x2(Frag<float>& f, const float* p0, const float* p1) {
  const float4 a = *reinterpret_cast<const float4*>(p0);
  const float4 b = *reinterpret_cast<const float4*>(p1);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

__device__ __forceinline__ f32x4 mma(const Frag<bf16>& a, const Frag<bf16>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<float>& a, const Frag<float>& b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace m3
