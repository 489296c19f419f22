// Shared device helpers for the gfx950 kernels of libtpshard.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define TP_LDS __attribute__((address_space(3)))

// ---- element conversion -------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// ---- exact GeLU and its derivative (fp32) ---------------------------------------------------------
// GeLU(x) = x·Φ(x), Φ(x) = ½(1 + erf(x/√2)); GeLU'(x) = Φ(x) + x·φ(x), φ(x) = exp(−x²/2)/√(2π).
// Φ comes from erfc(u) = (a1·t + a2·t² + a3·t³ + a4·t⁴ + a5·t⁵)·exp(−u²), t = 1/(1 + p·u), u = |x|/√2
// ≥ 0 (Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26, |error| ≤ 1.5e-7),
// with Φ(x) = 1 − erfc(u)/2 for x ≥ 0 and erfc(u)/2 below: GeLU within 2.1e-7 and GeLU' within 7e-8
// of their exact values, about half the instructions of a general-purpose erf in the GEMM epilogues,
// and exp(−u²) = exp(−x²/2) is φ's factor as well.
struct NormalCdf {
  float Phi;   // Φ(x)
  float e;     // exp(−x²/2)
};
__device__ __forceinline__ NormalCdf normal_cdf(float x) {
  const float u = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, u, 1.0f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f),
                                      -0.284496736f), 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(x * x * -0.72134752044448170f);   // exp(−x²/2) = 2^(−x²/2·log2 e)
  const float h = 0.5f * poly * e;                                          // erfc(u) / 2
  return {x >= 0.0f ? 1.0f - h : h, e};
}
__device__ __forceinline__ float gelu_f(float x) { return x * normal_cdf(x).Phi; }
__device__ __forceinline__ float gelu_grad_f(float x) {
  const NormalCdf c = normal_cdf(x);
  return fmaf(x * 0.39894228040143268f, c.e, c.Phi);
}
// The tanh form ½x(1 + tanh(u)), u = √(2/π)(x + 0.044715x³); its derivative
// ½(1 + t) + ½x(1 − t²)·√(2/π)(1 + 3·0.044715x²), t = tanh(u) (tanhf from the device math library).
__device__ __forceinline__ float gelu_tanh_f(float x) {
  const float t = tanhf(0.79788456080286536f * (x + 0.044715f * x * x * x));
  return 0.5f * x * (1.0f + t);
}
__device__ __forceinline__ float gelu_tanh_grad_f(float x) {
  const float t = tanhf(0.79788456080286536f * (x + 0.044715f * x * x * x));
  return 0.5f * (1.0f + t) + 0.5f * x * (1.0f - t * t) * 0.79788456080286536f * (1.0f + 0.134145f * x * x);
}
// activation `act`: 0 the exact GeLU, 1 its tanh form (a uniform branch in the epilogues)
__device__ __forceinline__ float act_f(float x, int act) { return act ? gelu_tanh_f(x) : gelu_f(x); }
__device__ __forceinline__ float act_grad_f(float x, int act) { return act ? gelu_tanh_grad_f(x) : gelu_grad_f(x); }

// ---- matrix-core instructions (CDNA4) ------------------------------------------------------------
// 16x16x32 bf16: lane l supplies row (l % 16), k = 8*(l / 16) .. +7 of its operand; the result lane l
// holds D[4*(l / 16) + e][l % 16], e = 0..3.
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x4 fp32: lane l supplies row (l % 16), k = l / 16; same result layout.
__device__ __forceinline__ f32x4 mfma_16x16x4_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

}  // namespace tp
