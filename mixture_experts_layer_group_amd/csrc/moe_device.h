// Device-side helpers shared by the MoE layer kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// erfc by Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26:
// erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2), t = 1 / (1 + p x), x >= 0,
// |error| <= 1.5e-7.  At x = |z| / sqrt 2 this gives the normal tail
// Phi(-|z|) = erfc(|z| / sqrt 2) / 2 = (a1 t + ... + a5 t^5) / 2 exp(-z^2 / 2), which both
// GELU and its derivative need: the 1 / sqrt 2 is folded into p and the 1/2 into the a_i.
// az = |z|, e = exp(-z^2 / 2).  One hardware reciprocal (v_rcp_f32).
__device__ __forceinline__ float normal_tail_as7126(float az, float e) {
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752440f, az, 1.0f));
  float p = fmaf(0.5f * 1.061405429f, t, 0.5f * -1.453152027f);
  p = fmaf(p, t, 0.5f * 1.421413741f);
  p = fmaf(p, t, 0.5f * -0.284496736f);
  p = fmaf(p, t, 0.5f * 0.254829592f);
  return p * t * e;
}

// exp(-z^2 / 2) as one v_exp_f32 (a power of two) of z^2 (-log2(e) / 2).
__device__ __forceinline__ float exp_neg_half_sq(float z) {
  return __builtin_amdgcn_exp2f(z * z * -0.72134752044448170368f);
}

// GELU in its erf form, z Phi(z) = 0.5 z (1 + erf(z / sqrt 2)), written for both signs at
// once: z Phi(z) = max(z, 0) - |z| Phi(-|z|).
__device__ __forceinline__ float gelu_erf(float z) {
  const float az = fabsf(z);
  return fmaf(-az, normal_tail_as7126(az, exp_neg_half_sq(z)), fmaxf(z, 0.0f));
}

// GELU'(z) = Phi(z) + z phi(z), phi(z) = exp(-z^2 / 2) / sqrt(2 pi): the density's exponential
// is the one the tail uses.
__device__ __forceinline__ float gelu_grad(float z) {
  const float e = exp_neg_half_sq(z);
  const float q = normal_tail_as7126(fabsf(z), e);
  const float Phi = z > 0.0f ? 1.0f - q : q;
  return fmaf(z * 0.39894228040143267794f, e, Phi);
}

// Swish with beta = 1: z * sigmoid(z) = z / (1 + exp(-z)) (exp(-z) = inf for very negative z
// gives -0).
__device__ __forceinline__ float swish(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// d/dz z sigmoid(z) = sigmoid(z) (1 + z (1 - sigmoid(z))).
__device__ __forceinline__ float swish_grad(float z) {
  const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
  return s * (1.0f + z * (1.0f - s));
}

__device__ __forceinline__ float apply_act(float z, int act) {
  if (act == 0) return fmaxf(z, 0.0f);
  if (act == 1) return gelu_erf(z);
  return z;
}

// Cross-lane steps inside one 16-lane DPP row: swap neighbours
// (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1), mirror within 8 lanes, mirror within
// 16 lanes.  Each step pairs every lane with one other lane of its aligned group of 2, 4, 8,
// 16, so after log2(N) steps of a commutative combine every lane of an aligned group of N
// holds the group's total, the same bits in every lane.  DPP moves are VALU operations; the
// LDS-routed ds_bpermute of a generic shuffle costs an LDS round trip per step.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(dpp_i<CTRL>(static_cast<int>(u & 0xffffffffu)));
  const uint32_t hi = static_cast<uint32_t>(dpp_i<CTRL>(static_cast<int>(u >> 32)));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// Reductions over aligned groups of N <= 16 lanes.
template <int N>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  if (N > 2) v = fmaxf(v, dpp_f<kDppXor2>(v));
  if (N > 4) v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  if (N > 8) v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  if (N > 2) v += dpp_f<kDppXor2>(v);
  if (N > 4) v += dpp_f<kDppHalfMirror>(v);
  if (N > 8) v += dpp_f<kDppMirror>(v);
  return v;
}
template <int N>
__device__ __forceinline__ double group_sum(double v) {
  v += dpp_d<kDppXor1>(v);
  if (N > 2) v += dpp_d<kDppXor2>(v);
  if (N > 4) v += dpp_d<kDppHalfMirror>(v);
  if (N > 8) v += dpp_d<kDppMirror>(v);
  return v;
}
// Best (value, index) over the group: larger value, ties to the lower index.
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& bv, int& bi) {
  const float ov = dpp_f<CTRL>(bv);
  const int oi = dpp_i<CTRL>(bi);
  if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}
template <int N>
__device__ __forceinline__ void group_argmax(float& bv, int& bi) {
  argmax_step<kDppXor1>(bv, bi);
  if (N > 2) argmax_step<kDppXor2>(bv, bi);
  if (N > 4) argmax_step<kDppHalfMirror>(bv, bi);
  if (N > 8) argmax_step<kDppMirror>(bv, bi);
}

// Lanes of a wave with an index below this lane.
__device__ __forceinline__ uint64_t lanes_below() {
  const uint32_t lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

}  // namespace moe
