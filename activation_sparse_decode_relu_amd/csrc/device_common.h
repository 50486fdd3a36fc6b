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
// Plain (cache-allocating) loads, for the batched kernel's 256-byte operand runs: neighbouring
// runs of a row share cache lines.
__device__ __forceinline__ u32x4 ld_cached(const u32x4* p) { return *p; }

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

// The EPC vector elements matching one 16-byte weight chunk, held in registers.
template <int WT, int VT>
struct XChunk {
  static constexpr int WORDS = WFmt<WT>::EPC * (int)sizeof(typename VecT<VT>::T) / 4;
  unsigned w[WORDS];
  __device__ __forceinline__ void load(const typename VecT<VT>::T* p) {
    if constexpr (WORDS == 2) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(p);
      w[0] = v.x;
      w[1] = v.y;
    } else {
#pragma unroll
      for (int k = 0; k < WORDS / 4; ++k) {
        const u32x4 v = reinterpret_cast<const u32x4*>(p)[k];
        w[4 * k] = v.x;
        w[4 * k + 1] = v.y;
        w[4 * k + 2] = v.z;
        w[4 * k + 3] = v.w;
      }
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int k = 0; k < WORDS; ++k) w[k] = 0u;
  }
  __device__ __forceinline__ float f(int k) const { return __builtin_bit_cast(float, w[k]); }
};

// acc += sum over the chunk's elements of w_e * x_e   (q4: the group scale applied once)
template <int WT, int VT>
__device__ __forceinline__ void dot_chunk(float& acc, u32x4 w, const XChunk<WT, VT>& x, float scale);

template <>
__device__ __forceinline__ void dot_chunk<DT_F16, DT_F16>(float& acc, u32x4 w, const XChunk<DT_F16, DT_F16>& x,
                                                          float) {
  acc = fdot2u(w.x, x.w[0], acc);
  acc = fdot2u(w.y, x.w[1], acc);
  acc = fdot2u(w.z, x.w[2], acc);
  acc = fdot2u(w.w, x.w[3], acc);
}

template <>
__device__ __forceinline__ void dot_chunk<DT_F32, DT_F32>(float& acc, u32x4 w, const XChunk<DT_F32, DT_F32>& x,
                                                          float) {
  const f32x4 wv = __builtin_bit_cast(f32x4, w);
  acc = fmaf(wv.x, x.f(0), acc);
  acc = fmaf(wv.y, x.f(1), acc);
  acc = fmaf(wv.z, x.f(2), acc);
  acc = fmaf(wv.w, x.f(3), acc);
}

template <>
__device__ __forceinline__ void dot_chunk<DT_F16, DT_F32>(float& acc, u32x4 w, const XChunk<DT_F16, DT_F32>& x,
                                                          float) {
  const unsigned ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const f16x2 h = as_h2(ws[p]);
    acc = fmaf((float)h.x, x.f(2 * p), acc);
    acc = fmaf((float)h.y, x.f(2 * p + 1), acc);
  }
}

template <>
__device__ __forceinline__ void dot_chunk<DT_F32, DT_F16>(float& acc, u32x4 w, const XChunk<DT_F32, DT_F16>& x,
                                                          float) {
  const f32x4 wv = __builtin_bit_cast(f32x4, w);
  f16x2 h = as_h2(x.w[0]);
  acc = fmaf(wv.x, (float)h.x, acc);
  acc = fmaf(wv.y, (float)h.y, acc);
  h = as_h2(x.w[1]);
  acc = fmaf(wv.z, (float)h.x, acc);
  acc = fmaf(wv.w, (float)h.y, acc);
}

// int4 group of 32: acc += s * sum_e q_e x_e.  q_e * x_e is exact in fp32 (fp16 x small int).
template <>
__device__ __forceinline__ void dot_chunk<DT_Q4, DT_F16>(float& acc, u32x4 w, const XChunk<DT_Q4, DT_F16>& x,
                                                         float scale) {
  float g = 0.f;
  const unsigned words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const unsigned q = words[k] ^ 0x88888888u;
    g = fdot2(q4pair(q), as_h2(x.w[4 * k]), g);
    g = fdot2(q4pair(q >> 8), as_h2(x.w[4 * k + 1]), g);
    g = fdot2(q4pair(q >> 16), as_h2(x.w[4 * k + 2]), g);
    g = fdot2(q4pair(q >> 24), as_h2(x.w[4 * k + 3]), g);
  }
  acc = fmaf(g, scale, acc);
}

template <>
__device__ __forceinline__ void dot_chunk<DT_Q4, DT_F32>(float& acc, u32x4 w, const XChunk<DT_Q4, DT_F32>& x,
                                                         float scale) {
  float g = 0.f;
  const unsigned words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const unsigned nib = (words[k] >> (4 * e)) & 0xFu;
      const int q = (int)nib - (int)((nib & 0x8u) << 1);
      g = fmaf((float)q, x.f(8 * k + e), g);
    }
  }
  acc = fmaf(g, scale, acc);
}

// Sum over the 64 lanes, returned uniformly to every lane.  Within each row
// of 16 lanes, DPP swaps (adjacent lanes, adjacent pairs, half-row mirror, row
// mirror) leave the row total, bitwise identical, in all 16 lanes; the four
// row totals are then added in a fixed order.  No LDS traffic.
template <int CTRL>
__device__ __forceinline__ float dpp_shuffled(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_shuffled<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_shuffled<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_shuffled<0x141>(v);  // row_half_mirror
  v += dpp_shuffled<0x140>(v);  // row_mirror
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float v) { return (f16)v; }

}  // namespace pik
