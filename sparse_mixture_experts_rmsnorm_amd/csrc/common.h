// Device helpers shared by the HIP kernels of libmoe_mi355x (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Native 16-byte vector (HIP's uint4 is a struct that can defeat SROA when
// kept in arrays, sending them to scratch or LDS).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 with round-to-nearest-even: gfx950's v_cvt_pk_bf16_f32
// (NaN stays NaN).  pk_bf16 converts a pair in one instruction, a in the
// low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// element <-> float for the two storage types (float, or bf16 bits)
__device__ __forceinline__ float tof(float v) { return v; }
__device__ __forceinline__ float tof(uint16_t v) { return bf2f(v); }
template <typename T> __device__ __forceinline__ T fromf(float v);
template <> __device__ __forceinline__ float fromf<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t fromf<uint16_t>(float v) { return f2bf(v); }

// elements per 16-byte vector
template <typename T> struct Vec16 { static constexpr int N = 16 / sizeof(T); };

__device__ __forceinline__ void unpack16(const uint4& v, float* o, const float*) {
  o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
  o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack16(const uint4& v, float* o, const uint16_t*) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ uint4 pack16(const float* o, const float*) {
  return make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                    __float_as_uint(o[3]));
}
__device__ __forceinline__ uint4 pack16(const float* o, const uint16_t*) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pk_bf16(o[2 * i], o[2 * i + 1]);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// erf(x) by Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.26:
// 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2), t = 1 / (1 + p x)
// for x >= 0, odd in x; |error| <= 1.5e-7 absolute (about 2.5 fp32 ulp near
// 1), with the hardware exp2 and reciprocal: a dozen instructions where the
// library erff takes about thirty, which matters in the GEMM epilogues (128
// values per lane per tile, not overlapped with the MFMAs).
__device__ __forceinline__ float erf_as7126(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.0f));
  float p = fmaf(1.061405429f, t, -1.453152027f);
  p = fmaf(p, t, 1.421413741f);
  p = fmaf(p, t, -0.284496736f);
  p = fmaf(p, t, 0.254829592f);
  p *= t;
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * ax * ax);
  return copysignf(fmaf(-p, e, 1.0f), x);
}
__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erf_as7126(z * 0.70710678118654752f));
}
__device__ __forceinline__ float gelu_tanh(float z) {
  const float c = 0.79788456080286536f;  // sqrt(2/pi)
  return 0.5f * z * (1.0f + tanhf(c * (z + 0.044715f * z * z * z)));
}
// 1 / (1 + e^-z) by the hardware exp2 and reciprocal (about 2 ulp)
__device__ __forceinline__ float sigmoidf(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}
__device__ __forceinline__ float silu(float z) { return z * sigmoidf(z); }

// Derivatives (the backward pass): GELU' = Phi(z) + z phi(z); the tanh
// form's derivative with u = c (z + 0.044715 z^3); SiLU' = s (1 + z (1 - s)).
__device__ __forceinline__ float gelu_erf_grad(float z) {
  return 0.5f * (1.0f + erff(z * 0.70710678118654752f)) +
         z * 0.39894228040143268f * expf(-0.5f * z * z);
}
__device__ __forceinline__ float gelu_tanh_grad(float z) {
  const float c = 0.79788456080286536f;
  const float t = tanhf(c * (z + 0.044715f * z * z * z));
  return 0.5f * (1.0f + t) + 0.5f * z * (1.0f - t * t) * c * (1.0f + 0.134145f * z * z);
}

// Set bits of a wave-uniform lane mask in the lanes below this one (the
// lane's rank among the set lanes), by the mbcnt pair: two instructions,
// where a popcount of the mask ANDed with a per-lane mask of the lower lanes
// takes a 64-bit AND and two counts.
__device__ __forceinline__ int rank_below(uint64_t mask) {
  return int(__builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32),
                                       __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u)));
}

// Wave-wide sum (all 64 lanes get the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace moe
