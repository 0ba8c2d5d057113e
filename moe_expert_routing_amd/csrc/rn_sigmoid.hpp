// rn_sigmoid.hpp - correctly rounded binary32 sigmoid for gfx950.
//
// The router scores are s = sigma(x) = 1 / (1 + e^-x) (a sigmoid router,
// "[ROCm][Perf] Kimi-K3: token-sharded residual stream for long prefills",
// author's reply on shard-routed test coverage). Expert selection compares
// s + bias exactly, so s must not depend on how sigma is evaluated: it is the
// binary32 value nearest to the real sigma(x).
//
// Method (Ziv's strategy):
//   1. evaluate sigma in binary64 with relative error below 2^-50;
//   2. round to binary32; if the binary64 value lies within 2^-44 (relative)
//      of a binary32 rounding boundary, re-evaluate in double-double
//      arithmetic (error below 2^-95) and round that.
// sigma(x) for finite nonzero binary32 x is transcendental
// (Lindemann-Weierstrass), so it is never exactly a rounding boundary.
//
// All code here is compiled with -ffp-contract=off: the error-free
// transformations (TwoSum, TwoProduct) rely on each operation being rounded
// on its own. FMAs are written explicitly where intended.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ln 2 = LN2_A + LN2_B + LN2_C with |rest| < 2^-143. LN2_A has 32 significant
// bits, so n * LN2_A is exact for |n| < 2^21.
constexpr double LN2_A = 0x1.62e42ff000000p-1;
constexpr double LN2_B = -0x1.718432a1b0e26p-35;
constexpr double LN2_C = -0x1.9ff0342542fc3p-90;
constexpr double INV_LN2 = 0x1.71547652b82fep+0;

// Above this x, 1 - sigma(x) < 2^-57 and sigma rounds to 1.0f; below the
// negative bound, sigma(x) < e^-110 < 2^-158 and rounds to +0.
constexpr float SIG_ONE_ABOVE = 40.0f;
constexpr float SIG_ZERO_BELOW = -110.0f;

// e^y for y in [-110, 0]: y = n ln2 + r, |r| <= ln2/2 (+tiny), e^r by its
// Taylor series to degree 13 (truncation < 2^-57), then scaled by 2^n.
// Relative error below 2^-51.
__device__ __forceinline__ double exp_nonpos_f64(double y) {
  const double n = __builtin_rint(y * INV_LN2);
  double r = __builtin_fma(-n, LN2_A, y);  // exact
  r = __builtin_fma(-n, LN2_B, r);
  double p = 1.0 / 6227020800.0;           // 1/13!
  p = __builtin_fma(p, r, 1.0 / 479001600.0);
  p = __builtin_fma(p, r, 1.0 / 39916800.0);
  p = __builtin_fma(p, r, 1.0 / 3628800.0);
  p = __builtin_fma(p, r, 1.0 / 362880.0);
  p = __builtin_fma(p, r, 1.0 / 40320.0);
  p = __builtin_fma(p, r, 1.0 / 5040.0);
  p = __builtin_fma(p, r, 1.0 / 720.0);
  p = __builtin_fma(p, r, 1.0 / 120.0);
  p = __builtin_fma(p, r, 1.0 / 24.0);
  p = __builtin_fma(p, r, 1.0 / 6.0);
  p = __builtin_fma(p, r, 0.5);
  p = __builtin_fma(p, r, 1.0);
  p = __builtin_fma(p, r, 1.0);
  return __builtin_ldexp(p, (int)n);
}

// sigma(x) in binary64, |x| within the bounds above.
__device__ __forceinline__ double sigmoid_f64(float x) {
  const double y = -__builtin_fabs((double)x);
  const double e = exp_nonpos_f64(y);
  const double den = 1.0 + e;
  return (x >= 0.0f) ? 1.0 / den : e / den;
}

// ---------------------------------------------------------------------------
// Double-double arithmetic (Dekker 1971; Knuth, TAOCP vol. 2, 4.2.2):
// a value is h + l with |l| <= ulp(h)/2.
// ---------------------------------------------------------------------------
struct dd {
  double h, l;
};

__device__ __forceinline__ dd two_sum(double a, double b) {
  const double s = a + b;
  const double bb = s - a;
  const double e = (a - (s - bb)) + (b - bb);
  return {s, e};
}

__device__ __forceinline__ dd fast_two_sum(double a, double b) {  // |a| >= |b|
  const double s = a + b;
  return {s, b - (s - a)};
}

__device__ __forceinline__ dd two_prod(double a, double b) {
  const double p = a * b;
  return {p, __builtin_fma(a, b, -p)};
}

__device__ __forceinline__ dd dd_add(dd a, dd b) {
  dd s = two_sum(a.h, b.h);
  const dd t = two_sum(a.l, b.l);
  s.l += t.h;
  s = fast_two_sum(s.h, s.l);
  s.l += t.l;
  return fast_two_sum(s.h, s.l);
}

__device__ __forceinline__ dd dd_neg(dd a) { return {-a.h, -a.l}; }

__device__ __forceinline__ dd dd_mul(dd a, dd b) {
  dd p = two_prod(a.h, b.h);
  p.l += a.h * b.l + a.l * b.h;
  return fast_two_sum(p.h, p.l);
}

__device__ __forceinline__ dd dd_mul_d(dd a, double b) {
  dd p = two_prod(a.h, b);
  p.l += a.l * b;
  return fast_two_sum(p.h, p.l);
}

// a / b for a double b (long division with an exact remainder).
__device__ __forceinline__ dd dd_div_d(dd a, double b) {
  const double q1 = a.h / b;
  const dd p = two_prod(q1, b);
  const double rem = ((a.h - p.h) - p.l) + a.l;
  const double q2 = rem / b;
  return fast_two_sum(q1, q2);
}

// a / b (three quotient digits).
__device__ __forceinline__ dd dd_div(dd a, dd b) {
  const double q1 = a.h / b.h;
  dd r = dd_add(a, dd_neg(dd_mul_d(b, q1)));
  const double q2 = r.h / b.h;
  r = dd_add(r, dd_neg(dd_mul_d(b, q2)));
  const double q3 = r.h / b.h;
  dd q = fast_two_sum(q1, q2);
  return dd_add(q, dd{q3, 0.0});
}

// Nearest binary32 to the double-double value s = h + l (s > 0). Only when h
// is exactly halfway between two binary32 values does l decide.
__device__ __forceinline__ float dd_to_f32(dd s) {
  float f = (float)s.h;
  const double fd = (double)f;
  if (fd != s.h) {
    const uint32_t u = __float_as_uint(f);
    const double nb = (s.h > fd) ? (double)__uint_as_float(u + 1u)
                                 : (u == 0u ? -1.0 : (double)__uint_as_float(u - 1u));
    const double m = 0.5 * (fd + nb);
    if (s.h == m && ((s.l > 0.0 && nb > fd) || (s.l < 0.0 && nb < fd))) f = (float)nb;
  }
  return f;
}

// sigma(x) rounded to binary32 through double-double evaluation.
__device__ __noinline__ float sigmoid_rn32_dd(float x) {
  if (x > SIG_ONE_ABOVE) return 1.0f;
  if (x < SIG_ZERO_BELOW) return 0.0f;
  const double y = -__builtin_fabs((double)x);
  const double n = __builtin_rint(y * INV_LN2);
  const double r0 = __builtin_fma(-n, LN2_A, y);  // exact
  dd r = dd_add(dd{r0, 0.0}, dd_neg(two_prod(n, LN2_B)));
  r = dd_add(r, dd{-n * LN2_C, 0.0});
  // e^r = 1 + r (1 + r/2 (1 + r/3 (1 + ...))), 26 levels (truncation < 2^-140)
  dd p = {1.0, 0.0};
  for (int k = 26; k >= 1; --k) {
    p = dd_div_d(dd_mul(p, r), (double)k);
    p = dd_add(p, dd{1.0, 0.0});
  }
  const int ni = (int)n;
  const dd e = {__builtin_ldexp(p.h, ni), __builtin_ldexp(p.l, ni)};
  const dd den = dd_add(e, dd{1.0, 0.0});
  const dd s = (x >= 0.0f) ? dd_div(dd{1.0, 0.0}, den) : dd_div(e, den);
  return dd_to_f32(s);
}

// Relative distance to a binary32 rounding boundary below which the binary64
// value is re-evaluated.
constexpr double ZIV_REL = 0x1p-44;

// Nearest binary32 to d in [0, 1]; `risky` is set when d lies within
// ZIV_REL * d of the boundary between two binary32 values.
__device__ __forceinline__ float rn32_checked(double d, bool &risky) {
  const float f = (float)d;
  const uint32_t u = __float_as_uint(f);
  const double fd = (double)f;
  const double m_up = 0.5 * (fd + (double)__uint_as_float(u + 1u));
  const double m_dn = (u == 0u) ? -1.0 : 0.5 * (fd + (double)__uint_as_float(u - 1u));
  const double thr = ZIV_REL * d;
  risky = (m_up - d <= thr) || (d - m_dn <= thr);
  return f;
}

// The binary32 nearest to sigma(x), for every finite binary32 x.
__device__ __forceinline__ float sigmoid_rn32(float x) {
  if (x > SIG_ONE_ABOVE) return 1.0f;
  if (x < SIG_ZERO_BELOW) return 0.0f;
  bool risky;
  float f = rn32_checked(sigmoid_f64(x), risky);
  if (risky) f = sigmoid_rn32_dd(x);
  return f;
}

// Two sigmoids at once: the two binary64 evaluations are independent, so
// their latencies overlap (same results as sigmoid_rn32 on each input).
__device__ __forceinline__ void sigmoid_rn32_x2(float x0, float x1, float &f0, float &f1) {
  const float c0 = fminf(fmaxf(x0, SIG_ZERO_BELOW), SIG_ONE_ABOVE);
  const float c1 = fminf(fmaxf(x1, SIG_ZERO_BELOW), SIG_ONE_ABOVE);
  bool r0, r1;
  f0 = rn32_checked(sigmoid_f64(c0), r0);
  f1 = rn32_checked(sigmoid_f64(c1), r1);
  if (r0) f0 = sigmoid_rn32_dd(c0);
  if (r1) f1 = sigmoid_rn32_dd(c1);
  f0 = x0 > SIG_ONE_ABOVE ? 1.0f : (x0 < SIG_ZERO_BELOW ? 0.0f : f0);
  f1 = x1 > SIG_ONE_ABOVE ? 1.0f : (x1 < SIG_ZERO_BELOW ? 0.0f : f1);
}

}  // namespace moe
