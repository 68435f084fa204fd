// The rotation of one rotate-half RoPE pair, shared by the RoPE kernel and
// the Phase-1 kernel that rotates Q itself, so both produce the same bits.
//
// The angle pos * theta_j reaches ~1e6 rad at million-token positions, where
// an fp32 product is off by up to ~5e-2 rad.  It is formed and reduced
// modulo 2*pi in fp64 (two-constant Cody-Waite step), so the fp32 angle
// handed to sincosf is within ~1e-7 rad of the exact one.
#pragma once
#include <hip/hip_runtime.h>

namespace star {

__device__ __forceinline__ void rope_angle(double pos, double inv_freq, float& c, float& s) {
  constexpr double kTwoPiHi = 6.283185307179586;          // fp64(2*pi)
  constexpr double kTwoPiLo = 2.4492935982947064e-16;     // 2*pi - kTwoPiHi
  constexpr double kInvTwoPi = 0.15915494309189535;
  const double ang = pos * inv_freq;
  const double k = rint(ang * kInvTwoPi);
  double r = fma(-k, kTwoPiHi, ang);
  r = fma(-k, kTwoPiLo, r);
  sincosf((float)r, &s, &c);
}

// (x1, x2) -> (x1 c - x2 s, x2 c + x1 s), each with one explicit fma
__device__ __forceinline__ void rope_rotate(float x1, float x2, float c, float s, float& y1,
                                            float& y2) {
  y1 = __builtin_fmaf(x1, c, -(x2 * s));
  y2 = __builtin_fmaf(x2, c, x1 * s);
}

}  // namespace star
