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

// Δ in base-2 units: Δ' = Δ·log2(e).  With Δ = softplus(x) = ln(1 + e^x),
//   Δ' = log2(1 + 2^t),  t = x·log2(e),
// so the decay is Ā = e^{ΔA} = 2^{Δ'A} (one v_exp_f32 of Δ'·A, no scale) and the
// input term Δ·u·B = Δ'·u·(B·ln 2) once B is staged pre-scaled by ln 2.
// For t >= 25, 1 + 2^t rounds to 2^t and the log returns t; the clamp keeps 2^t
// finite and the max restores Δ' = t beyond it.  Where 1 + 2^t rounds (t << 0),
// Δ' carries an absolute error below 2^-24, i.e. a negligible absolute
// perturbation of Ā and of Δ·u·B.
__device__ __forceinline__ float softplus_log2(float x) {
  const float t = x * kLog2e;
  return __builtin_fmaxf(t, lg2(1.0f + ex2(__builtin_fminf(t, 64.0f))));
}

// Exact zero-order hold of the input term: B̄u = ((e^{ΔA} - 1)/A)·B·u = Δ·φ(ΔA)·B·u
// with φ(x) = (e^x - 1)/x (φ(0) = 1, the A = 0 limit).  From the decay a = e^x
// already computed, (a - 1)·(1/A) is accurate while |x| is not small; below
// |x| = 1/16 the subtraction would cancel, and φ comes from its Taylor series
// 1 + x/2 + x²/6 + x³/24 + x⁴/120, whose remainder there is below 2^-30.
// Arguments: a = e^x, x = ΔA, dt = Δ, inv_a = 1/A (any value when A = 0).
__device__ __forceinline__ float zoh_coef(float a, float x, float dt, float inv_a) {
  const float direct = __builtin_fmaf(a, inv_a, -inv_a);
  const float series =
      __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 120.0f, 1.0f / 24.0f), 1.0f / 6.0f), 0.5f), 1.0f);
  return __builtin_fabsf(x) < 0.0625f ? dt * series : direct;
}

// The same coefficient from base-2 arguments, as the forward scan holds them:
// t = Δ'·A with Δ' = Δ·log2 e (so ΔA = t·ln 2 and a = 2^t) and dl = Δ'.  The
// series Δ·φ(ΔA) becomes dl·Σ_m k_m t^m with k_m = ln2^(m+1)/(m+1)!, which
// saves the two conversions to natural units.  Three terms and the switch at
// |t| < 0.055 balance the two errors: the direct form's relative error is
// about ulp(a)/|a - 1| <= 2^-23/(0.055 ln 2) = 3.1e-6 above the switch (from
// the rounding of a itself), the series' truncation (ln2^3/24)·t^3 <= 2.3e-6
// below it.
__device__ __forceinline__ float zoh_coef_b2(float a, float t, float dl, float inv_a) {
  constexpr float k0 = 0.69314718056f;    // ln 2
  constexpr float k1 = 0.240226506959f;   // ln2^2 / 2
  constexpr float k2 = 0.0555041086648f;  // ln2^3 / 6
  const float direct = __builtin_fmaf(a, inv_a, -inv_a);
  const float series = __builtin_fmaf(t, __builtin_fmaf(t, k2, k1), k0);
  return __builtin_fabsf(t) < 0.055f ? dl * series : direct;
}

// Derivative of c = (e^{ΔA} - 1)/A with respect to A: (Δ·e^{ΔA} - c)/A.  For
// small |x| = |ΔA| the difference cancels; there the series of
// c = Δ·Σ_m x^m/(m+1)! differentiated term by term,
// Δ²·(1/2 + x/3 + x²/8 + x³/30 + x⁴/144), is used (Δ²/2 at A = 0).
__device__ __forceinline__ float zoh_coef_dA(float a, float x, float dt, float c, float inv_a) {
  const float direct = (dt * a - c) * inv_a;
  const float series = __builtin_fmaf(
      x, __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 144.0f, 1.0f / 30.0f), 0.125f), 1.0f / 3.0f),
      0.5f);
  return __builtin_fabsf(x) < 0.0625f ? dt * dt * series : direct;
}

// silu(z) = z·sigmoid(z) = z / (1 + e^{-z}); for z -> -inf, e^{-z} -> inf and
// the reciprocal gives 0.
__device__ __forceinline__ float silu_f(float z) { return z * rcp(1.0f + ex2(-z * kLog2e)); }

// ---- V (2, 4 or 8) consecutive channels of u / delta / z, kept as raw bits until used ----
template <typename T, int V>
struct Vec;

template <int V>
struct Vec<uint16_t, V> {  // bfloat16 bit patterns, V/2 dwords
  static_assert(V == 2 || V == 4 || V == 8, "2, 4 or 8 channels");
  uint32_t w[V / 2];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < V / 2; ++i) w[i] = 0;
  }
  __device__ __forceinline__ void load(const uint16_t* p) {
    if constexpr (V == 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (V == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      w[0] = v.x; w[1] = v.y;
    } else {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
  }
  __device__ __forceinline__ float get(int j) const {
    const uint32_t x = w[j >> 1];
    return __uint_as_float((j & 1) ? (x & 0xffff0000u) : (x << 16));
  }
};

template <int V>
struct Vec<float, V> {
  static_assert(V == 2 || V == 4 || V == 8, "2, 4 or 8 channels");
  float f[V];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < V; ++i) f[i] = 0.f;
  }
  __device__ __forceinline__ void load(const float* p) {
    if constexpr (V == 2) {
      const float2 v = *reinterpret_cast<const float2*>(p);
      f[0] = v.x; f[1] = v.y;
    } else {
#pragma unroll
      for (int i = 0; i < V / 4; ++i) {
        const float4 v = reinterpret_cast<const float4*>(p)[i];
        f[4 * i] = v.x; f[4 * i + 1] = v.y; f[4 * i + 2] = v.z; f[4 * i + 3] = v.w;
      }
    }
  }
  __device__ __forceinline__ float get(int j) const { return f[j]; }
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (v_cvt_pk_bf16_f32: round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <int V>
__device__ __forceinline__ void storeV(uint16_t* p, const float (&y)[V]) {
  if constexpr (V == 8) {
    uint4 v;
    v.x = pack_bf16x2(y[0], y[1]);
    v.y = pack_bf16x2(y[2], y[3]);
    v.z = pack_bf16x2(y[4], y[5]);
    v.w = pack_bf16x2(y[6], y[7]);
    *reinterpret_cast<uint4*>(p) = v;
  } else if constexpr (V == 4) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
  } else {
    *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(y[0], y[1]);
  }
}

template <int V>
__device__ __forceinline__ void storeV(float* p, const float (&y)[V]) {
  if constexpr (V == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(y[0], y[1]);
  } else {
#pragma unroll
    for (int i = 0; i < V / 4; ++i)
      reinterpret_cast<float4*>(p)[i] = make_float4(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]);
  }
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- E (1, 2 or 4) consecutive elements of B / C, kept as raw bits until used ----
template <typename T, int E>
struct Small;

template <>
struct Small<uint16_t, 4> {
  uint2 v;
  __device__ __forceinline__ void zero() { v = make_uint2(0, 0); }
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, 0);
    v = make_uint2(x[0], x[1]);
  }
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
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
    v = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]), __uint_as_float(x[3]));
  }
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

// ---- buffer-resource access: SGPR descriptor + scalar row offset + per-lane offset ----
// Raw buffer descriptor over `bytes` bytes at `base` (stride 0; word 3 as for gfx9 raw buffers).
// A buffer offset past every slice this library addresses through a
// descriptor (each at most 2^31 bytes, by the plans' limits): a raw buffer
// access there is out of range, so a store is dropped and a load returns 0.
// A descriptor of 0 bytes drops every access the same way.
constexpr uint32_t kDrop = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint16_t buf_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint16_t*) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ float buf_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float*) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ void buf_store(uint16_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void buf_store(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)voff, (int)soff, 0);
}
// Two adjacent channels of one token row: one 32-bit (bf16) or 64-bit (f32)
// buffer load, and the matching store of two results.
template <typename T>
struct Pair;
template <>
struct Pair<uint16_t> {
  uint32_t w;
  __device__ __forceinline__ void zero() { w = 0; }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    w = __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0);
  }
  __device__ __forceinline__ float get(int j) const { return __uint_as_float(j ? (w & 0xffff0000u) : (w << 16)); }
};
template <>
struct Pair<float> {
  u32x2 w;
  __device__ __forceinline__ void zero() { w = u32x2{0u, 0u}; }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    w = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, 0);
  }
  __device__ __forceinline__ float get(int j) const { return __uint_as_float(w[j]); }
};
__device__ __forceinline__ void store_pair(float y0, float y1, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint16_t*) {
  __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(y0, y1), r, (int)voff, 0, 0);
}
__device__ __forceinline__ void store_pair(float y0, float y1, __amdgpu_buffer_rsrc_t r, uint32_t voff, float*) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(y0), __float_as_uint(y1)}, r, (int)voff, 0, 0);
}

__device__ __forceinline__ uint16_t to_bf16(float y) { return (uint16_t)(pack_bf16x2(y, 0.0f) & 0xffffu); }
__device__ __forceinline__ void store_out(float y, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint16_t*) {
  buf_store(to_bf16(y), r, voff, soff);
}
__device__ __forceinline__ void store_out(float y, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float*) {
  buf_store(y, r, voff, soff);
}

__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float load1(const uint16_t* p) { return __uint_as_float(((uint32_t)*p) << 16); }
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ void store1(uint16_t* p, float y) {
  *p = (uint16_t)(pack_bf16x2(y, 0.0f) & 0xffffu);
}
__device__ __forceinline__ void store1(float* p, float y) { *p = y; }

}  // namespace mscan
