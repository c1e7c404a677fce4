// Device helpers shared by the gfx950 kernels of libhspec.so.
//
// Element types: `float` and `bf16_t` (raw bfloat16 bits).  Matrix-core work
// goes through one primitive, mma8(): a 16x16 output tile accumulated over 32
// contraction indices, where lane l supplies row/column (l % 16) and the eight
// contraction indices of group (l / 16).  For bf16 that is one
// v_mfma_f32_16x16x32_bf16; for fp32 it is eight v_mfma_f32_16x16x4_f32, one
// per element of the lane's group.  The result tile is laid out the gfx9 way:
// lane l holds column (l % 16) of rows 4*(l/16) .. 4*(l/16)+3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace hspec {

// f(std::integral_constant<int, I>{}) for I = B .. E-1: register-array
// indices derived from I are constants before any loop unrolling, so the
// arrays always live in registers.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

struct bf16_t {
  uint16_t bits;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
// Native 16-byte vector for register rings: arrays of it are split into
// registers, where arrays of the uint4 struct can end up in scratch.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

// Eight contraction-adjacent elements held by one lane.
template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
  uint4 v;  // 8 bf16, element e in half (e & 1) of dword (e >> 1)
};
template <> struct Vec8<float> {
  float v[8];
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// Two fp32 -> one dword of two bf16 (lo, hi), round to nearest even: a single
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{lo, hi}, bf16x2v));
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v.bits); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return bf16_t{f32_to_bf16(v)}; }

template <typename T> __device__ __forceinline__ void zero8(Vec8<T>& a);
template <> __device__ __forceinline__ void zero8<bf16_t>(Vec8<bf16_t>& a) { a.v = make_uint4(0, 0, 0, 0); }
template <> __device__ __forceinline__ void zero8<float>(Vec8<float>& a) {
#pragma unroll
  for (int e = 0; e < 8; ++e) a.v[e] = 0.f;
}

// 16-byte aligned load of 8 consecutive elements.
template <typename T> __device__ __forceinline__ void load8(Vec8<T>& a, const T* p);
template <> __device__ __forceinline__ void load8<bf16_t>(Vec8<bf16_t>& a, const bf16_t* p) {
  a.v = *reinterpret_cast<const uint4*>(p);
}
template <> __device__ __forceinline__ void load8<float>(Vec8<float>& a, const float* p) {
  const float4 x = reinterpret_cast<const float4*>(p)[0];
  const float4 y = reinterpret_cast<const float4*>(p)[1];
  a.v[0] = x.x; a.v[1] = x.y; a.v[2] = x.z; a.v[3] = x.w;
  a.v[4] = y.x; a.v[5] = y.y; a.v[6] = y.z; a.v[7] = y.w;
}

// 16x16 tile += A(16x32) * B(32x16), operand layout as described at the top.
template <typename T>
__device__ __forceinline__ f32x4 mma8(const Vec8<T>& a, const Vec8<T>& b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mma8<bf16_t>(const Vec8<bf16_t>& a, const Vec8<bf16_t>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, a.v),
                                                 __builtin_bit_cast(bf16x8v, b.v), c, 0, 0, 0);
}
// 32x32 output tile over 16 contraction indices, bf16 in, fp32 accumulate
// (v_mfma_f32_32x32x16_bf16): lane l supplies row/column (l % 32) and the
// eight contraction indices 8*(l/32) .. 8*(l/32)+7; result element i of lane
// l is column (l % 32), row 8*(i/4) + 4*(l/32) + (i%4).  One wave keeps this
// instruction at the matrix-core peak with as few as two accumulator chains.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mma32(const Vec8<bf16_t>& a, const Vec8<bf16_t>& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, a.v),
                                                 __builtin_bit_cast(bf16x8v, b.v), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mma8<float>(const Vec8<float>& a, const Vec8<float>& b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
  return c;
}

// Stores of fp32 results in the element type of an output tensor.
template <typename T> __device__ __forceinline__ void store_out(T* p, float v);
template <> __device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_out<bf16_t>(bf16_t* p, float v) { p->bits = f32_to_bf16(v); }

// four consecutive outputs (16-byte aligned fp32, 8-byte aligned bf16)
template <typename T> __device__ __forceinline__ void store_out4(T* p, float4 v);
template <> __device__ __forceinline__ void store_out4<float>(float* p, float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <> __device__ __forceinline__ void store_out4<bf16_t>(bf16_t* p, float4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

// Element e of a Vec8 as fp32 (used by register transposes and conversions).
__device__ __forceinline__ uint32_t half_of(uint32_t dw, int hi) { return hi ? (dw >> 16) : (dw & 0xFFFFu); }

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Wave-wide (64-lane) butterflies.
__device__ __forceinline__ float wave_xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m, 64)); }
__device__ __forceinline__ float wave_xor_sum(float v, int m) { return v + __shfl_xor(v, m, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float silu_f(float v) { return v / (1.f + __expf(-v)); }

// log(1 + e^v); above 20 the correction is below fp32 resolution.
__device__ __forceinline__ float softplus_f(float v) { return v > 20.f ? v : log1pf(__expf(v)); }

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace hspec
