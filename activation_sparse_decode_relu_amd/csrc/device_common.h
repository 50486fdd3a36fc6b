// Device-side building blocks shared by the gfx950 kernels: element formats,
// 16-byte streaming loads, per-chunk dot products and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pik {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

enum : int { DT_F32 = 0, DT_F16 = 1, DT_Q4 = 2 };

constexpr int WAVE = 64;

// Elements held by one 16-byte chunk of a weight row.
template <int WT> struct WFmt;
template <> struct WFmt<DT_F32> { static constexpr int EPC = 4; };
template <> struct WFmt<DT_F16> { static constexpr int EPC = 8; };
template <> struct WFmt<DT_Q4> { static constexpr int EPC = 32; };  // one int4 group

template <int VT> struct VecT;
template <> struct VecT<DT_F32> { using T = float; };
template <> struct VecT<DT_F16> { using T = f16; };

// Bytes of a row of K elements.
__host__ __device__ constexpr size_t row_bytes(int wt, size_t k) {
  return wt == DT_F32 ? k * 4 : (wt == DT_F16 ? k * 2 : k / 2);
}

// Weight rows are read exactly once per step: stream them past the caches.
__device__ __forceinline__ u32x4 ld_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ u32x2 ld_stream(const u32x2* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ f16x2 as_h2(unsigned v) { return __builtin_bit_cast(f16x2, v); }

__device__ __forceinline__ float fdot2(f16x2 a, f16x2 b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}
__device__ __forceinline__ float fdot2u(unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// Two int4 codes (bits 0-3 and 4-7 of t, two's complement) as exact fp16 values.
// (q ^ 8) is q + 8 in [0, 15]; placed in the mantissa of 1024.0 it reads 1024 + q + 8.
__device__ __forceinline__ f16x2 q4pair(unsigned t) {
  const unsigned hb = 0x64006400u | (t & 0xFu) | ((t & 0xF0u) << 12);
  const f16x2 bias = {(f16)1032.0f, (f16)1032.0f};
  return as_h2(hb) - bias;
}

// acc += sum over the chunk's elements of w_e * v_e   (v points at the chunk's first element)
template <int WT, int VT>
__device__ __forceinline__ void dot_chunk(float& acc, u32x4 w, const typename VecT<VT>::T* v, float scale);

template <>
__device__ __forceinline__ void dot_chunk<DT_F16, DT_F16>(float& acc, u32x4 w, const f16* v, float) {
  const u32x4 xv = *reinterpret_cast<const u32x4*>(v);
  acc = fdot2u(w.x, xv.x, acc);
  acc = fdot2u(w.y, xv.y, acc);
  acc = fdot2u(w.z, xv.z, acc);
  acc = fdot2u(w.w, xv.w, acc);
}

template <>
__device__ __forceinline__ void dot_chunk<DT_F32, DT_F32>(float& acc, u32x4 w, const float* v, float) {
  const f32x4 xv = *reinterpret_cast<const f32x4*>(v);
  const f32x4 wv = __builtin_bit_cast(f32x4, w);
  acc = fmaf(wv.x, xv.x, acc);
  acc = fmaf(wv.y, xv.y, acc);
  acc = fmaf(wv.z, xv.z, acc);
  acc = fmaf(wv.w, xv.w, acc);
}

template <>
__device__ __forceinline__ void dot_chunk<DT_F16, DT_F32>(float& acc, u32x4 w, const float* v, float) {
  const f32x4 x0 = *reinterpret_cast<const f32x4*>(v);
  const f32x4 x1 = *reinterpret_cast<const f32x4*>(v + 4);
  f16x2 h;
  h = as_h2(w.x); acc = fmaf((float)h.x, x0.x, acc); acc = fmaf((float)h.y, x0.y, acc);
  h = as_h2(w.y); acc = fmaf((float)h.x, x0.z, acc); acc = fmaf((float)h.y, x0.w, acc);
  h = as_h2(w.z); acc = fmaf((float)h.x, x1.x, acc); acc = fmaf((float)h.y, x1.y, acc);
  h = as_h2(w.w); acc = fmaf((float)h.x, x1.z, acc); acc = fmaf((float)h.y, x1.w, acc);
}

template <>
__device__ __forceinline__ void dot_chunk<DT_F32, DT_F16>(float& acc, u32x4 w, const f16* v, float) {
  const u32x2 xv = *reinterpret_cast<const u32x2*>(v);
  const f32x4 wv = __builtin_bit_cast(f32x4, w);
  f16x2 h;
  h = as_h2(xv.x); acc = fmaf(wv.x, (float)h.x, acc); acc = fmaf(wv.y, (float)h.y, acc);
  h = as_h2(xv.y); acc = fmaf(wv.z, (float)h.x, acc); acc = fmaf(wv.w, (float)h.y, acc);
}

// int4 group of 32: acc += s * sum_e q_e v_e.  q_e * v_e is exact in fp32 (fp16 x small int).
template <>
__device__ __forceinline__ void dot_chunk<DT_Q4, DT_F16>(float& acc, u32x4 w, const f16* v, float scale) {
  const u32x4* xp = reinterpret_cast<const u32x4*>(v);
  float g = 0.f;
  const unsigned words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const u32x4 xv = xp[k];
    const unsigned q = words[k] ^ 0x88888888u;
    g = fdot2(q4pair(q), as_h2(xv.x), g);
    g = fdot2(q4pair(q >> 8), as_h2(xv.y), g);
    g = fdot2(q4pair(q >> 16), as_h2(xv.z), g);
    g = fdot2(q4pair(q >> 24), as_h2(xv.w), g);
  }
  acc = fmaf(g, scale, acc);
}

template <>
__device__ __forceinline__ void dot_chunk<DT_Q4, DT_F32>(float& acc, u32x4 w, const float* v, float scale) {
  float g = 0.f;
  const unsigned words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(v + 8 * k);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(v + 8 * k + 4);
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = (int)((words[k] >> (4 * e)) & 0xFu) - (int)(((words[k] >> (4 * e)) & 0x8u) << 1);
      g = fmaf((float)q, xs[e], g);
    }
  }
  acc = fmaf(g, scale, acc);
}

// Sum over the 64 lanes; every lane returns lane 0's result (one fixed association order).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, WAVE);
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float v) { return (f16)v; }

}  // namespace pik
