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

// pi/2 split in two doubles (head + tail) for argument reduction, and 2/pi.
constexpr double kHalfPiHi = 1.570796326794896558;
constexpr double kHalfPiLo = 6.123233995736766036e-17;
constexpr double kTwoOverPi = 0.63661977236758134308;

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

// cos and sin of pos * omega.  The angle a is formed and reduced in fp64
// (at position 32768 an fp32 angle would already be off by ~2e-3 rad):
// n = rint(a * 2/pi), r = a - n * pi/2 with pi/2 in two parts, so
// |r| <= pi/4 and the quadrant is n mod 4.  sin r and cos r then come from
// their Taylor series in fp32, through r^9 and r^8 (the first omitted terms,
// r^11/11! and r^10/10!, stay below 3e-8 for |r| <= pi/4), and the quadrant
// swaps and negates them.  A library sincosf would also carry its own
// large-argument reduction, which the compiler evaluates on every call.
__device__ __forceinline__ void rope_cos_sin(double pos, double omega, float& c, float& s) {
  const double a = pos * omega;
  const double n = rint(a * kTwoOverPi);
  double rd = fma(-n, kHalfPiHi, a);
  rd = fma(-n, kHalfPiLo, rd);
  const float r = (float)rd, r2 = r * r;
  float sr = fmaf(r2, 1.0f / 362880.0f, -1.0f / 5040.0f);
  sr = fmaf(r2, sr, 1.0f / 120.0f);
  sr = fmaf(r2, sr, -1.0f / 6.0f);
  sr = fmaf(r2 * r, sr, r);
  float cr = fmaf(r2, 1.0f / 40320.0f, -1.0f / 720.0f);
  cr = fmaf(r2, cr, 1.0f / 24.0f);
  cr = fmaf(r2, cr, -0.5f);
  cr = fmaf(r2, cr, 1.0f);
  const int q = (int)(int64_t)n & 3;   // two's complement: also right for n < 0
  const float sv = (q & 1) ? cr : sr, cv = (q & 1) ? sr : cr;
  s = (q & 2) ? -sv : sv;
  c = ((q + 1) & 2) ? -cv : cv;
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
