// Device helpers shared by the libcsa kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ------------------------------------------------------------------ FP8 E4M3 (OCP)
// Decode by definition: bias 7, subnormals m * 2^-9, S.1111.111 = NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v;
  if (e == 15u && m == 7u) v = __uint_as_float(0x7fc00000u);
  else if (e == 0u) v = static_cast<float>(m) * 0x1p-9f;
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -v : v;
}

// Round to nearest even, saturating at +-448; NaN -> 0x7f.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  float a = fabsf(x);
  if (!(a == a)) return 0x7fu;
  if (a >= 448.0f) return sign | 0x7eu;
  int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xffu) - 127;
  if (e < -6) {                                   // subnormal spacing 2^-9
    const uint32_t q = static_cast<uint32_t>(rintf(a * 0x1p9f));   // 0..8; 8 is the min normal code
    return sign | q;
  }
  float q = rintf(ldexpf(a, 3 - e));             // in [8, 16]
  if (q >= 16.0f) { q = 8.0f; e += 1; }
  const uint32_t code = (static_cast<uint32_t>(e + 7) << 3) | (static_cast<uint32_t>(q) - 8u);
  return sign | (code > 0x7eu ? 0x7eu : code);
}

// ------------------------------------------------------------------ E2M1 (OCP MX)
// Round to nearest even on {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating at +-6.
__device__ __forceinline__ uint32_t f32_to_e2m1(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 28) & 0x8u;
  const float a = fabsf(x);
  if (!(a == a)) return 0x7u | sign;
  if (a < 1.0f) {
    const uint32_t q = static_cast<uint32_t>(rintf(a * 2.0f));     // 0, 1 or 2 (2 = 1.0)
    return sign | q;
  }
  if (a >= 6.0f) return sign | 0x7u;
  int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xffu) - 127;   // 0, 1, 2
  float q = rintf(ldexpf(a, 1 - e));                                   // in [2, 4]
  if (q >= 4.0f) { q = 2.0f; e += 1; }
  if (e > 2) return sign | 0x7u;
  return sign | (static_cast<uint32_t>(e + 1) << 1) | (static_cast<uint32_t>(q) - 2u);
}

__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float v = e == 0u ? 0.5f * static_cast<float>(m)
                          : ldexpf(1.0f + 0.5f * static_cast<float>(m), static_cast<int>(e) - 1);
  return (c & 8u) ? -v : v;
}

// ------------------------------------------------------------------ raw buffer loads
// A buffer descriptor over [base, base + bytes): a load whose byte offset is
// at or past `bytes` returns 0 without touching memory (the buffer range
// check), so ragged tails need neither a branch nor a clamped address.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}
__device__ __forceinline__ uint32_t buf_load_u32(buf_rsrc r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(byte_off), 0, 0);
}

// A value the caller knows to be equal on every lane of the wave, moved to
// scalar registers (so what is derived from it stays scalar).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Load of a value the whole wave reads at one address, through the scalar
// data cache (constant address space: the kernel never writes it).
__device__ __forceinline__ int64_t scalar_load(const int64_t* p, int64_t i) {
  typedef const __attribute__((address_space(4))) int64_t c64;
  return ((c64*)(p))[i];
}

// ------------------------------------------------------------------ wave reductions
// Butterfly over the 64 lanes; the order of operations is fixed by the lane
// pattern, so every lane ends with the same bits on every run.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// RoPE rotation of pair i at absolute position pos: angle = pos * theta_i with
// theta_i = base^(-2i/R) precomputed in double on the host.  The product and
// the reduction to [-pi, pi] run in double, so positions up to 2^24 and beyond
// keep full float accuracy in sin / cos.
__device__ __forceinline__ void rope_sincos(int64_t pos, double theta, float* s, float* c) {
  const double two_pi = 6.283185307179586476925286766559;
  const double ang = static_cast<double>(pos) * theta;
  const double red = fma(-rint(ang * (1.0 / two_pi)), two_pi, ang);
  sincosf(static_cast<float>(red), s, c);
}

// Host-side RoPE frequency table: theta_i = base^(-2i/R), i < R/2.
constexpr int kMaxRopePairs = 64;
inline void fill_rope_theta(double* theta, int R, float base) {
  for (int i = 0; i < kMaxRopePairs; ++i)
    theta[i] = (R > 0 && i < R / 2) ? pow(static_cast<double>(base), -2.0 * i / R) : 0.0;
}

}  // namespace csa
