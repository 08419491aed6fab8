// device_math.h -- gfx950 device helpers of the selective-scan kernels:
// hardware transcendentals, softplus, silu, and 8-wide bf16/f32 loads and
// stores.  exp/log come straight from the CDNA hardware instructions
// (v_exp_f32 is 2^x, v_log_f32 is log2 x, v_rcp_f32 is 1/x); the functions
// built on them are derived here from their definitions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mscan {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^{-|x|}).
// With e = e^{-|x|} in (0, 1] and s = fl(1 + e), the rounding error of s is
// r = e - (s - 1) exactly (Fast2Sum, since 1 >= e), and
// log1p(e) = log(s) + log(1 + r/s) = log(s) + r + O(r^2 + r(s-1)),
// an absolute error below 2^-25; the plain log(1 + e) would lose every bit of
// e below 2^-24 and give Δ a relative error up to 2^-24/e for negative x.
__device__ __forceinline__ float softplus_f(float x) {
  const float e = ex2(-__builtin_fabsf(x) * kLog2e);
  const float s = 1.0f + e;
  const float r = e - (s - 1.0f);
  return __builtin_fmaxf(x, 0.0f) + __builtin_fmaf(lg2(s), kLn2, r);
}

// silu(z) = z·sigmoid(z) = z / (1 + e^{-z}); for z -> -inf, e^{-z} -> inf and
// the reciprocal gives 0.
__device__ __forceinline__ float silu_f(float z) { return z * rcp(1.0f + ex2(-z * kLog2e)); }

// ---- 8 consecutive elements of u / delta / z (16 B of bf16, 32 B of f32) ----
template <typename T>
struct Vec8;

template <>
struct Vec8<uint16_t> {  // bfloat16 bit patterns
  uint4 v;
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float get(int j) const {
    const uint32_t w = (j >> 1) == 0 ? v.x : (j >> 1) == 1 ? v.y : (j >> 1) == 2 ? v.z : v.w;
    return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};

template <>
struct Vec8<float> {
  float4 a, b;
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ float get(int j) const {
    switch (j) {
      case 0: return a.x; case 1: return a.y; case 2: return a.z; case 3: return a.w;
      case 4: return b.x; case 5: return b.y; case 6: return b.z; default: return b.w;
    }
  }
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (v_cvt_pk_bf16_f32: round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ void store8(uint16_t* p, const float (&y)[8]) {
  uint4 v;
  v.x = pack_bf16x2(y[0], y[1]);
  v.y = pack_bf16x2(y[2], y[3]);
  v.z = pack_bf16x2(y[4], y[5]);
  v.w = pack_bf16x2(y[6], y[7]);
  *reinterpret_cast<uint4*>(p) = v;
}

__device__ __forceinline__ void store8(float* p, const float (&y)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(y[0], y[1], y[2], y[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(y[4], y[5], y[6], y[7]);
}

// ---- E (1, 2 or 4) consecutive elements of B / C, kept as raw bits until used ----
template <typename T, int E>
struct Small;

template <>
struct Small<uint16_t, 4> {
  uint2 v;
  __device__ __forceinline__ void zero() { v = make_uint2(0, 0); }
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t w = e < 2 ? v.x : v.y;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <>
struct Small<uint16_t, 2> {
  uint32_t v;
  __device__ __forceinline__ void zero() { v = 0; }
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ float get(int e) const {
    return __uint_as_float((e & 1) ? (v & 0xffff0000u) : (v << 16));
  }
};
template <>
struct Small<uint16_t, 1> {
  uint32_t v;
  __device__ __forceinline__ void zero() { v = 0; }
  __device__ __forceinline__ void load(const uint16_t* p) { v = *p; }
  __device__ __forceinline__ float get(int) const { return __uint_as_float(v << 16); }
};
template <>
struct Small<float, 4> {
  float4 v;
  __device__ __forceinline__ void zero() { v = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ float get(int e) const { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }
};
template <>
struct Small<float, 2> {
  float2 v;
  __device__ __forceinline__ void zero() { v = make_float2(0.f, 0.f); }
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float2*>(p); }
  __device__ __forceinline__ float get(int e) const { return e == 0 ? v.x : v.y; }
};
template <>
struct Small<float, 1> {
  float v;
  __device__ __forceinline__ void zero() { v = 0.f; }
  __device__ __forceinline__ void load(const float* p) { v = *p; }
  __device__ __forceinline__ float get(int) const { return v; }
};

__device__ __forceinline__ float load1(const uint16_t* p) { return __uint_as_float(((uint32_t)*p) << 16); }
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ void store1(uint16_t* p, float y) {
  *p = (uint16_t)(pack_bf16x2(y, 0.0f) & 0xffffu);
}
__device__ __forceinline__ void store1(float* p, float y) { *p = y; }

}  // namespace mscan
