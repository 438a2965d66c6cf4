// kda_common.hpp -- shared device helpers for the gfx950 KDA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr float kLog2e = 1.4426950408889634f;

// Native clang vector types (usable with the nontemporal builtins).
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 is carried as raw 16-bit patterns; arithmetic is always fp32.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Typed scalar load/store of the two supported element types.
template <typename T> struct io;
template <> struct io<float> {
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float x) { p[i] = x; }
};
template <> struct io<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i].bits); }
  __device__ __forceinline__ static void store(bf16_t* p, int64_t i, float x) { p[i].bits = f32_to_bf16(x); }
};

// Hardware 2^x (v_exp_f32) and reciprocal (v_rcp_f32), both ~1 ulp.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Bounded gate in log2 units: g2 = (g_min * log2 e) * sigmoid(exp(A) z).
// `ea_l2e` = exp(A) * log2 e, `gmin_l2e` = g_min * log2 e.
// sigmoid(x) = 1 / (1 + 2^(-x log2 e)); 2^(+large) = inf gives sigmoid 0.
__device__ __forceinline__ float gate_log2(float z, float ea_l2e, float gmin_l2e) {
  float e = fast_exp2(-ea_l2e * z);
  return gmin_l2e * fast_rcp(1.0f + e);
}

// Fused prologue ("Kimi K3: the paper and proofs side by side", section 2.1.1,
// Equations 2-6): q and k are divided by sqrt(|x|^2 + 1e-6); the write
// strength beta in (0, 1) comes from its logit through the logistic sigmoid.
constexpr float kL2Eps = 1e-6f;
__device__ __forceinline__ float rsqrt_fast(float x) { return __builtin_amdgcn_rsqf(x); }  // v_rsq_f32, ~1 ulp
__device__ __forceinline__ float sigmoid_fast(float x) { return fast_rcp(1.0f + fast_exp2(-x * kLog2e)); }

}  // namespace kda
