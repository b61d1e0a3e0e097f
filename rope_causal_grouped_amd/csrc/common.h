// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 2*pi split in two doubles (head + tail) for argument reduction.
constexpr double kTwoPiHi = 6.283185307179586232;
constexpr double kTwoPiLo = 2.449293598294706414e-16;
constexpr double kInvTwoPi = 0.15915494309189533577;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// Round-to-nearest-even float -> bf16 bit pattern.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// RoPE parameters of a call.  Pair j turns by pos * omega_j with
// omega_j = theta^(-2j/d); with YaRN scaling by a factor s, omega_j is blended
// towards omega_j / s by a ramp over the pair index (0 at or below ramp_lo:
// kept; 1 at or above ramp_hi: divided by s), and cos and sin are multiplied
// by mscale.  inv_factor = 1 and mscale = 1 give plain RoPE.
struct RopeParams {
  double log2_theta;
  double inv_factor;
  double ramp_lo, ramp_hi;
  float mscale;
};

// RoPE inverse frequency of pair j, in fp64.
__device__ __forceinline__ double rope_omega(int j, int d, const RopeParams& rp) {
  const double w = exp2(-(2.0 * (double)j / (double)d) * rp.log2_theta);
  if (rp.inv_factor == 1.0) return w;
  const double r = fmin(fmax(((double)j - rp.ramp_lo) / (rp.ramp_hi - rp.ramp_lo), 0.0), 1.0);
  return w * (1.0 - r) + w * rp.inv_factor * r;
}

// cos and sin of pos * omega.  The angle is formed and reduced to
// [-pi, pi] in fp64 (at position 32768 an fp32 angle would already be off
// by ~2e-3 rad), then evaluated in fp32.
__device__ __forceinline__ void rope_cos_sin(double pos, double omega, float& c,
                                             float& s) {
  double a = pos * omega;
  double n = rint(a * kInvTwoPi);
  double r = fma(-n, kTwoPiHi, a);
  r = fma(-n, kTwoPiLo, r);
  sincosf((float)r, &s, &c);
}

// cos and sin of pair j at position pos under rp (YaRN's mscale included).
__device__ __forceinline__ void rope_cs(double pos, int j, int d, const RopeParams& rp, float& c,
                                        float& s) {
  rope_cos_sin(pos, rope_omega(j, d, rp), c, s);
  c *= rp.mscale;
  s *= rp.mscale;
}

// Power of two that score operands with largest magnitude amax are divided
// by before rounding to fp16: 0 below 2^14, else the smallest e with
// amax * 2^-e < 2^14, so the operands stay finite (fp16 ends at 65504).
__device__ __forceinline__ int kexp_of(float amax) {
  if (!(amax >= 16384.0f)) return 0;
  int e;
  (void)frexpf(amax, &e);   // amax < 2^e
  return e - 14;
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

// v_permlane32_swap exchanges the upper half-wave of its first operand with
// the lower half-wave of its second; with both operands = v, the two results
// hold, in every lane, v of that lane and v of lane ^ 32 (in some order).
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace gqa
