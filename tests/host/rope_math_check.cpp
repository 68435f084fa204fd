// Host checks of the fp64 RoPE arithmetic the kernels share (rope_math.h,
// compiled here for the host).
//
// 1. star::sincos_cw against long double (x87, 64-bit significand)
//    sinl/cosl, over the angles RoPE produces (position x theta_j up to
//    past 2^20 rad) and next to multiples of pi/2.  A rotated value is
//    x1 c - x2 s with |c|, |s| <= 1, so what bounds its error is the
//    absolute error of c and s; the error in ulps is reported where
//    |value| >= 1/16.
// 2. star::f64_to_f32_for_bf16 followed by a nearest-even rounding of the
//    fp32 value to bf16, against a one-step nearest-even rounding of the
//    fp64 value done on its bits (integer arithmetic), on random values,
//    exact bf16 midpoints, values one fp64 ulp either side of a midpoint,
//    and values that round to an fp32 midpoint.
// Prints "max_abs max_ulp n_sincos bf16_mismatches n_bf16".
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>

#include "../../block_sparse_amd/csrc/rope_math.h"

static double ulp_err(double got, long double ref) {
  const double r = (double)ref;
  const double u = std::nextafter(std::fabs(r), INFINITY) - std::fabs(r);
  return (double)(std::fabs((long double)got - ref) / (long double)u);
}

// nearest-even bf16 of a finite fp64 value in fp32's normal range, from its
// bits: keep sign, exponent and 7 fraction bits, round on the other 45
static uint16_t bf16_ref(double d) {
  uint64_t b;
  std::memcpy(&b, &d, 8);
  const uint64_t sign = b >> 63;
  const int64_t e = (int64_t)((b >> 52) & 0x7ff) - 1023;
  uint64_t m = (b & ((1ull << 52) - 1)) | (1ull << 52);   // 53-bit significand
  const int sh = 45;
  uint64_t q = m >> sh, rem = m & ((1ull << sh) - 1), half = 1ull << (sh - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  int64_t ee = e;
  if (q == (1ull << 8)) { q >>= 1; ++ee; }
  const uint32_t be = (uint32_t)(ee + 127);
  return (uint16_t)((sign << 15) | (be << 7) | (q & 0x7f));
}

static uint16_t bf16_lib(double d) {
  const float f = star::f64_to_f32_for_bf16(d);
  uint32_t u;
  std::memcpy(&u, &f, 4);
  // nearest-even fp32 -> bf16 (what the device's conversion does)
  const uint32_t r = u + 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(r >> 16);
}

int main() {
  std::mt19937_64 g(12345);
  std::uniform_real_distribution<double> pos(0.0, 1100000.0);
  std::uniform_int_distribution<int> jd(0, 63);
  double mabs = 0, mulp = 0;
  long n = 0;
  auto acc = [&](double got, long double ref) {
    mabs = std::fmax(mabs, (double)std::fabs((long double)got - ref));
    if (std::fabs((double)ref) >= 0.0625) mulp = std::fmax(mulp, ulp_err(got, ref));
  };
  auto one = [&](double x) {
    double s, c;
    star::sincos_cw(x, s, c);
    acc(s, sinl((long double)x));
    acc(c, cosl((long double)x));
    ++n;
  };
  for (int t = 0; t < 2000000; ++t) {
    const double p = std::floor(pos(g));
    const double th = (double)std::pow(500000.0L, -2.0L * jd(g) / 128.0L);
    one(p * th);
  }
  for (int p = 0; p < 4096; ++p) one((double)p);
  for (int p = 1048576 - 2048; p < 1048576 + 2048; ++p) one((double)p);
  for (int k = 1; k < 200000; k += 7) {
    const double x = (double)(k * 1.5707963267948966192313216916397514L);
    one(x);
    one(std::nextafter(x, 0.0));
    one(std::nextafter(x, INFINITY));
  }

  long bad = 0, nb = 0;
  auto chk = [&](double d) {
    ++nb;
    if (bf16_lib(d) != bf16_ref(d)) ++bad;
  };
  std::normal_distribution<double> nd(0.0, 1.0);
  for (int t = 0; t < 2000000; ++t) chk(nd(g) * std::ldexp(1.0, (int)(g() % 40) - 20));
  std::uniform_int_distribution<uint32_t> hi(0x3c00, 0x43ff);  // bf16 with |x| in [2^-7, 2^8)
  for (int t = 0; t < 200000; ++t) {
    const uint32_t h = hi(g) | ((g() & 1) << 15);
    const uint32_t mid = (h << 16) | 0x8000u;                   // a bf16 rounding midpoint
    float fm;
    std::memcpy(&fm, &mid, 4);
    const double m = fm;
    chk(m);                                                    // exactly the midpoint
    chk(std::nextafter(m, 0.0));
    chk(std::nextafter(m, INFINITY));
    chk(std::nextafter(m, -INFINITY));
    // within half an fp32 ulp of the midpoint: rounds to it in fp32
    const double hu = std::ldexp(std::fabs(m), -25);
    chk(m + hu * 0.75);
    chk(m - hu * 0.75);
  }
  std::printf("%.3e %.3f %ld %ld %ld\n", mabs, mulp, n, bad, nb);
  return 0;
}
