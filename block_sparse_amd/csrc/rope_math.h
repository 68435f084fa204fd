// The rotation of one rotate-half RoPE pair, shared by every kernel that
// rotates (the RoPE and KV-append kernels, Phase 1 rotating Q itself, the
// fused decode step), so all of them store the same bits for a position.
//
// Everything up to the one rounding to the storage type is fp64:
//  * the angle is the IEEE product pos * theta_j (theta_j from the host, the
//    fp64 value nearest base^(-2j/D));
//  * its cos/sin come from sincos_cw below (error ~1-2 fp64 ulp);
//  * the rotated pair is x1 c - x2 s, x2 c + x1 s in fp64;
//  * the result is rounded once, to nearest even, to bf16 (or fp32).
// So a stored rotated value is the exact rotation rounded once, except
// where the fp64 value lies within a few fp64 ulps of a bf16 rounding
// midpoint (probability ~2^-44 per element).
//
// The functions are host-callable too, so a host test can measure
// sincos_cw against extended-precision references.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

namespace star {

// cos and sin of x in fp64.  Cody-Waite reduction by pi/2, x = k pi/2 + r,
// with pi/2 split in three parts: P1 and P2 carry 27 and 25 significant
// bits, so k P1 and k P2 are exact for |k| < 2^26, and x - k P1 is exact
// (Sterbenz); P3 holds the next 53 bits (P1 + P2 + P3 is pi/2 to within
// 5e-35).  Then the Taylor series of sin and cos on |r| <= pi/4, through
// r^17 and r^18 (truncation below 1e-19), and the quadrant k mod 4.  The
// constants are pi/2 rounded to 27 bits, the rest rounded to 25 bits, the
// rest to 53 bits, and 1/n!.  Beyond |x| = 2^25 (positions past ~3e7 at
// theta_0 = 1) the device library's sincos is used instead.
__host__ __device__ __forceinline__ void sincos_cw(double x, double& s, double& c) {
  constexpr double kTwoOverPi = 0.6366197723675814;
  constexpr double P1 = 1.570796325802803;        // 0x1.921fb54p+0
  constexpr double P2 = 9.920935739593517e-10;    // 0x1.10b461p-30
  constexpr double P3 = 5.721188726109832e-18;    // 0x1.a62633145c06ep-58
  if (__builtin_expect(!(__builtin_fabs(x) < 33554432.0), 0)) {
#if defined(__HIP_DEVICE_COMPILE__)
    sincos(x, &s, &c);
#else
    s = std::sin(x);
    c = std::cos(x);
#endif
    return;
  }
  const double k = __builtin_rint(x * kTwoOverPi);
  double r = __builtin_fma(-k, P1, x);
  r = __builtin_fma(-k, P2, r);
  r = __builtin_fma(-k, P3, r);
  const double z = r * r;
  // sin r = r + r z (S3 + z (S5 + ... + z S17))
  double ps = -1.0 / 355687428096000.0;                 // -1/17!
  ps = __builtin_fma(ps, z, 1.0 / 1307674368000.0);     //  1/15!
  ps = __builtin_fma(ps, z, -1.0 / 6227020800.0);       // -1/13!
  ps = __builtin_fma(ps, z, 1.0 / 39916800.0);          //  1/11!
  ps = __builtin_fma(ps, z, -1.0 / 362880.0);           // -1/9!
  ps = __builtin_fma(ps, z, 1.0 / 5040.0);              //  1/7!
  ps = __builtin_fma(ps, z, -1.0 / 120.0);              // -1/5!
  ps = __builtin_fma(ps, z, 1.0 / 6.0);                 //  1/3! (sign below)
  const double sr = __builtin_fma(-(r * z), ps, r);
  // cos r = 1 + z (C2 + z (C4 + ... + z C18))
  double pc = -1.0 / 6402373705728000.0;                // -1/18!
  pc = __builtin_fma(pc, z, 1.0 / 20922789888000.0);    //  1/16!
  pc = __builtin_fma(pc, z, -1.0 / 87178291200.0);      // -1/14!
  pc = __builtin_fma(pc, z, 1.0 / 479001600.0);         //  1/12!
  pc = __builtin_fma(pc, z, -1.0 / 3628800.0);          // -1/10!
  pc = __builtin_fma(pc, z, 1.0 / 40320.0);             //  1/8!
  pc = __builtin_fma(pc, z, -1.0 / 720.0);              // -1/6!
  pc = __builtin_fma(pc, z, 1.0 / 24.0);                //  1/4!
  pc = __builtin_fma(pc, z, -0.5);                      // -1/2!
  const double cr = __builtin_fma(z, pc, 1.0);
  // quadrant: (c, s) = (cr, sr), (-sr, cr), (-cr, -sr), (sr, -cr)
  const int q = (int)(int64_t)k & 3;
  const double a = (q & 1) ? sr : cr;
  const double b = (q & 1) ? cr : sr;
  c = (q == 1 || q == 2) ? -a : a;
  s = (q >= 2) ? -b : b;
}

// cos and sin (fp64) of the angle pos * inv_freq
__host__ __device__ __forceinline__ void rope_cs(double pos, double inv_freq, double& c,
                                                 double& s) {
  sincos_cw(pos * inv_freq, s, c);
}

// (x1, x2) -> (x1 c - x2 s, x2 c + x1 s) in fp64
__host__ __device__ __forceinline__ void rope_rotate64(double x1, double x2, double c, double s,
                                                       double& y1, double& y2) {
  y1 = __builtin_fma(x1, c, -(x2 * s));
  y2 = __builtin_fma(x2, c, x1 * s);
}

// fp64 -> bf16 with one rounding to nearest even.  The fp64 value is first
// rounded to fp32 (nearest even) and that to bf16.  The two steps give the
// one-step result unless the fp32 value lands exactly on a bf16 rounding
// midpoint (low 16 bits 0x8000) while the fp64 value was not that
// midpoint: rounding is monotonic and every bf16 midpoint is an fp32
// value, so otherwise both lie on the same side of every midpoint.  In that
// rare case (~2^-16 of values) the fp32 value is moved one fp32 ulp toward
// the fp64 value before the second rounding.
__host__ __device__ __forceinline__ float f64_to_f32_for_bf16(double d) {
  const float f = (float)d;
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (__builtin_expect((u & 0xffffu) == 0x8000u, 0)) {
    const double back = (double)f;
    if (back != d) u += (__builtin_fabs(d) > __builtin_fabs(back)) ? 1u : 0xffffffffu;
  }
  return __builtin_bit_cast(float, u);
}

__device__ __forceinline__ __bf16 f64_to_bf16(double d) { return (__bf16)f64_to_f32_for_bf16(d); }

// two fp64 values -> a packed bf16 pair (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16_f64(double lo, double hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)f64_to_f32_for_bf16(lo), (__bf16)f64_to_f32_for_bf16(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace star
