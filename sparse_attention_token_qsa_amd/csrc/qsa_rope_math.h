// Rotary cos/sin in f32 with a certificate for their bf16 rounding.
//
// Host and device code: the kernels use it through qsa_device.h, and a CPU
// test (tests/host/rope_f32_check.cpp) evaluates the same code on every
// position the library accepts to check the error bound below.  Uses only
// correctly rounded IEEE operations (fmaf, rintf, products and sums with
// contraction off), so host and device give the same bits.
#pragma once

#include <cmath>
#include <cstdint>

#if defined(__HIP__)
#define QSA_HD __host__ __device__
#else
#define QSA_HD
#endif

namespace qsa {

// cos and sin of a float angle with |a| < 2^18, in f32.
//   Reduction (Cody and Waite, "Software Manual for the Elementary
//   Functions", 1980): k = nearest integer to a * 2/pi, r = a - k pi/2 with
//   pi/2 split into three f32 parts.  The first FMA is exact: for |a| >= 1,
//   a and k * P1 are multiples of 2^-23 and their difference is below 1 in
//   magnitude; below 1, k is 0 or 1 and the difference is a multiple of
//   2^-24.  The next two FMAs round once each.
//   Polynomials: the Taylor series of sin r to r^11 and of cos r to r^12
//   (coefficients 1/n! rounded to f32), Horner form; the first omitted terms
//   are below 7e-12 and 4e-13 on |r| <= pi/4.
// Absolute error of either result below 2^-22.7 by that analysis; the
// largest error seen over every position below 2^18 + 3 at the rotary
// frequencies of theta 1e4, 5e5, 1e7 and 123.5 is 2^-23.74.
QSA_HD inline void cos_sin_f32(float a, float& c, float& s) {
#if defined(__clang__)
#pragma clang fp contract(off)
#endif
  const float k = rintf(a * 0.636619747f);
  float r = fmaf(-k, 1.57079637f, a);           // pi/2, first 24 bits
  r = fmaf(-k, -4.37113883e-08f, r);             // next 24 bits
  r = fmaf(-k, -1.71512451e-15f, r);             // next 24 bits
  const float r2 = r * r;
  float ps = fmaf(r2, -2.50521079e-08f, 2.75573188e-06f);  // -1/11!, 1/9!
  ps = fmaf(ps, r2, -1.98412701e-04f);                     // -1/7!
  ps = fmaf(ps, r2, 8.33333377e-03f);                      // 1/5!
  ps = fmaf(ps, r2, -1.66666672e-01f);                     // -1/3!
  const float sr = fmaf(r * r2, ps, r);
  float pc = fmaf(r2, 2.08767559e-09f, -2.75573188e-07f);  // 1/12!, -1/10!
  pc = fmaf(pc, r2, 2.48015876e-05f);                      // 1/8!
  pc = fmaf(pc, r2, -1.38888892e-03f);                     // -1/6!
  pc = fmaf(pc, r2, 4.16666679e-02f);                      // 1/4!
  pc = fmaf(pc, r2, -0.5f);                                // -1/2!
  const float cr = fmaf(r2, pc, 1.0f);
  const int q = static_cast<int>(k) & 3;
  const float c0 = (q & 1) ? sr : cr;
  const float s0 = (q & 1) ? cr : sr;
  c = (q == 1 || q == 2) ? -c0 : c0;
  s = (q & 2) ? -s0 : s0;
}

// Error allowance for cos_sin_f32: its bound 2^-22.7 plus half an f32 ulp of
// a value below 1 (the reference rounds the exact value to f32 first), 2^-22.43
// together, with a factor above 1.3 to spare.  Every f32 angle the kernels
// evaluate this way has been checked against it (worst error 2^-23.70).
constexpr float kTrigSettle = 0x1p-22f;

// True when every real within err of v rounds to the same bf16 as v (round
// to nearest even): v is farther than err from the rounding midpoint of its
// bf16 interval (v and that midpoint share sign and exponent, so their
// difference is exact), and |v| >= 1024 err, which keeps v's bf16 spacing
// at least 4 err so that no other midpoint, including the one a quarter
// spacing below a power of two, lies within err.
QSA_HD inline bool bf16_rounding_settled(float v, float err) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const float mid = __builtin_bit_cast(float, (u & 0xFFFF0000u) | 0x8000u);
  return fabsf(v) >= 1024.0f * err && fabsf(v - mid) > err;
}

}  // namespace qsa
