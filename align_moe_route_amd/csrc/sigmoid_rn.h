// Correctly rounded FP32 logistic sigmoid, s = RN32(1 / (1 + e^-x)).
//
// The route-sort path converts router logits to FP32 and scores them with the
// sigmoid (page "Kimi-K3 B1 route-sort + prepared-MoE handoff (stack)",
// Summary); the library fixes that score as the correctly rounded FP32 value,
// so ids and weights do not depend on how an exp was implemented.
//
// Evaluation, for FP32 x:
//   * |x| < 2^-10: the series 1/2 + x/4 - x^3/48 + x^5/480, split into an
//     exact head 1/2 + x/4 and a tail, and the rounding side read off their
//     sum (float64 cannot see the cubic term next to 1/2 there, and 1/2 + x/4
//     is itself an FP32 rounding midpoint for many inputs);
//   * otherwise r = 1 / (1 + exp(-x)) in float64.  Its relative error is a few
//     units of 2^-53 (exp within an ulp, then one rounded add and one
//     correctly rounded divide), so RN32(r) is the correctly rounded result
//     unless r lies within that error of the midpoint between two FP32
//     neighbours.  Such inputs (about one in 2^19 at the window used, 2^-44
//     relative: r (1 - 2^-44) and r (1 + 2^-44) round to different FP32
//     values) are recomputed in double-double arithmetic (about 2^-100
//     relative) and the side of the midpoint is read from that value.
//
// Double-double exp: -x = n ln2 + r with ln2 split into three doubles (the
// first with 45 fractional bits, so n * L1 is exact for |n| <= 255), e^r from
// the nested Taylor form 1 + r(1 + r/2(1 + r/3(...(1 + r/25)))) (|r| < 0.35,
// so the first omitted term is below 2^-115), scaled by 2^n; then 1 / (1 + e)
// by one Newton correction of the float64 quotient.
//
// Host and device use the same code (the host build serves CPU checks of the
// refinement); every step is an IEEE operation spelled out in the source, with
// fma() where an exact product or remainder is needed.
#ifndef MOE_SIGMOID_RN_H
#define MOE_SIGMOID_RN_H

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

namespace sigrn {

struct dd {
  double hi, lo;
};

__host__ __device__ __forceinline__ uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}
__host__ __device__ __forceinline__ float f32_from(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// s + e = a + b exactly (Knuth)
__host__ __device__ __forceinline__ dd two_sum(double a, double b) {
  const double s = a + b;
  const double bb = s - a;
  const double e = (a - (s - bb)) + (b - bb);
  return {s, e};
}
// s + e = a + b exactly when |a| >= |b| (Dekker)
__host__ __device__ __forceinline__ dd quick_two_sum(double a, double b) {
  const double s = a + b;
  return {s, b - (s - a)};
}
__host__ __device__ __forceinline__ dd dd_add(dd a, dd b) {
  dd s = two_sum(a.hi, b.hi);
  const dd t = two_sum(a.lo, b.lo);
  s.lo += t.hi;
  s = quick_two_sum(s.hi, s.lo);
  s.lo += t.lo;
  return quick_two_sum(s.hi, s.lo);
}
__host__ __device__ __forceinline__ dd dd_mul(dd a, dd b) {
  const double p = a.hi * b.hi;
  const double e = fma(a.hi, b.hi, -p);  // exact error of the product
  return quick_two_sum(p, e + (a.hi * b.lo + a.lo * b.hi));
}
// a / n for a small positive integer n: the remainder of the first quotient is
// exact (fma), the second quotient carries the rest
__host__ __device__ __forceinline__ dd dd_div_small(dd a, double n) {
  const double q1 = a.hi / n;
  const double rem = fma(-q1, n, a.hi);
  const double q2 = (rem + a.lo) / n;
  return quick_two_sum(q1, q2);
}

// ln 2 = L1 + L2 + L3 (+ under 2^-150); L1 has 45 fractional bits.
constexpr double kLn2_1 = 0x1.62e42fefa3a00p-1;
constexpr double kLn2_2 = -0x1.0ca86c3898d00p-49;
constexpr double kLn2_3 = 0x1.f97b57a079a19p-103;

// 1 / (1 + e^-x) in double-double, for 2^-10 <= |x| <= 128.
__host__ __device__ inline dd sigmoid_dd(double x) {
  const double y = -x;
  const double n = rint(y * 1.4426950408889634);  // nearest integer to y / ln 2
  dd r = two_sum(y, -n * kLn2_1);                  // n * L1 exact
  const double p2 = n * kLn2_2;
  r = dd_add(r, dd{-p2, -fma(n, kLn2_2, -p2)});
  r = dd_add(r, dd{-n * kLn2_3, 0.0});
  dd e{1.0, 0.0};
  for (int j = 25; j >= 1; --j) e = dd_add(dd{1.0, 0.0}, dd_mul(dd_div_small(r, (double)j), e));
  const int ni = (int)n;
  e.hi = ldexp(e.hi, ni);
  e.lo = ldexp(e.lo, ni);
  const dd d = dd_add(dd{1.0, 0.0}, e);
  const double q1 = 1.0 / d.hi;
  double rem = fma(-q1, d.hi, 1.0);  // exact remainder of the float64 quotient
  rem -= q1 * d.lo;
  return quick_two_sum(q1, rem / d.hi);
}

// The double-double sigmoid of xd against the midpoint of the adjacent FP32
// values dn < up picks one of them.  Callers reach it about once in 2^19
// evaluations.
__host__ __device__ __forceinline__ float rn32_resolve(double xd, float dn, float up) {
  const dd s = sigmoid_dd(xd);
  const double mid = 0.5 * ((double)dn + (double)up);  // exact
  const double side = (s.hi - mid) + s.lo;             // s.hi - mid is exact (Sterbenz)
  if (side > 0.0) return up;
  if (side < 0.0) return dn;
  return (f32_bits(up) & 1u) ? dn : up;
}

// RN32 of the float64 sigmoid of an FP32 x, and whether it may differ from
// the correctly rounded value.  The float64 quotient r is within a relative
// 2^-44 of the exact value (several times its error bound), and rounding is
// monotonic, so when RN32(r (1 - 2^-44)) and RN32(r (1 + 2^-44)) agree, that
// is the correctly rounded result; otherwise `amb` is set, they are the two
// adjacent candidates `dn` < `up`, and rn32_resolve picks one.  Inputs with
// |x| < 2^-10 are resolved exactly here (series) and never set `amb`; NaN
// never sets it; for |x| > 128 it is never set, so the double-double range of
// rn32_resolve covers every input that sets it.
__host__ __device__ __forceinline__ float sigmoid_rn32_try(float x, bool& amb, float& up) {
  const double xd = (double)x;
  if (fabs(xd) < 0x1p-10) {
    amb = false;
    const double hi = 0.5 + 0.25 * xd;  // exact for |x| >= 2^-28; else far from a midpoint
    const double x2 = xd * xd;
    const double lo = xd * x2 * (-1.0 / 48.0 + x2 * (1.0 / 480.0));
    const float f = (float)hi;
    const double fb = (double)f;
    if (fb == hi) return f;
    const uint32_t fu = f32_bits(f);
    const float gg = f32_from(fb > hi ? fu - 1u : fu + 1u);  // other neighbour of hi
    const double gb = (double)gg;
    const double md = 0.5 * (fb + gb);
    const double d = (hi - md) + lo;  // side of the midpoint the exact value lies on
    const float u = fb > gb ? f : gg;
    const float dnv = fb > gb ? gg : f;
    if (d > 0.0) return u;
    if (d < 0.0) return dnv;
    return (f32_bits(u) & 1u) ? dnv : u;
  }
  const double r = 1.0 / (1.0 + exp(-xd));
  const float dn = (float)(r * (1.0 - 0x1p-44));
  up = (float)(r * (1.0 + 0x1p-44));
  amb = dn < up;
  return dn;
}

// Correctly rounded FP32 sigmoid of an FP32 x (round to nearest even).
__host__ __device__ __forceinline__ float sigmoid_rn32(float x) {
  bool amb;
  float up;
  const float dn = sigmoid_rn32_try(x, amb, up);
  if (amb) return rn32_resolve((double)x, dn, up);
  return dn;
}

}  // namespace sigrn

#endif  // MOE_SIGMOID_RN_H
