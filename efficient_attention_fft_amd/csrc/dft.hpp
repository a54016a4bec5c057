// dft.hpp -- in-register discrete Fourier transforms for gfx950 kernels.
//
// Small complex DFTs whose size is a compile-time constant R.  Every index is
// known at compile time, so the whole transform unrolls into straight-line
// VGPR code: radix-2, -3 and -4 butterflies; for a power of two R >= 8 a
// radix-2 decimation in time whose twiddled butterflies are written for
// fused multiply-add (6 instructions instead of 8; 32 points: 388 instead of
// 420); for other composite R a decimation-in-time split R = F * Q (Q-point
// transforms of the F interleaved subsequences, a twiddle
// exp(sign 2 pi i f k / R), then F-point transforms).  The twiddle constants
// are computed at compile time in double precision and rounded once to
// binary32.
//
// SIGN = -1 is the forward transform X[f] = sum_n x[n] exp(-2 pi i f n / R);
// SIGN = +1 is the unscaled inverse.
#pragma once

#include <hip/hip_runtime.h>

namespace spectre {

// ------------------------------------------------------------------ complex

__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
// a * conj(b)
__device__ __forceinline__ float2 cmulc(float2 a, float2 b) {
  return make_float2(a.x * b.x + a.y * b.y, a.y * b.x - a.x * b.y);
}
__device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
__device__ __forceinline__ float2 cscale(float2 a, float s) { return make_float2(a.x * s, a.y * s); }
// multiply by SIGN * i
template <int SIGN>
__device__ __forceinline__ float2 rot90(float2 a) {
  return SIGN > 0 ? make_float2(-a.y, a.x) : make_float2(a.y, -a.x);
}

// --------------------------------------------------- compile-time twiddles

namespace ct {

constexpr double kPi = 3.14159265358979323846264338327950288;

// Taylor series on |x| <= pi/4; 14 terms reach double rounding.
constexpr double sin_small(double x) {
  double x2 = x * x, term = x, sum = x;
  for (int i = 1; i < 14; ++i) {
    term *= -x2 / double((2 * i) * (2 * i + 1));
    sum += term;
  }
  return sum;
}
constexpr double cos_small(double x) {
  double x2 = x * x, term = 1.0, sum = 1.0;
  for (int i = 1; i < 14; ++i) {
    term *= -x2 / double((2 * i - 1) * (2 * i));
    sum += term;
  }
  return sum;
}

struct cd {
  double re, im;
};

// exp(sign * 2 pi i num / den): the angle is split exactly (integer
// arithmetic) into a nearest quarter turn plus a residual of at most pi/4.
constexpr cd expi(long num, long den, int sign) {
  num %= den;
  if (num < 0) num += den;
  long q = (4 * num + den / 2) / den;
  long r = 4 * num - q * den;
  double phi = (kPi / 2) * double(r) / double(den);
  double c = cos_small(phi), s = sin_small(phi);
  cd v{0.0, 0.0};
  switch (q & 3) {
    case 0: v = cd{c, s}; break;
    case 1: v = cd{-s, c}; break;
    case 2: v = cd{-c, -s}; break;
    default: v = cd{s, -c}; break;
  }
  v.im *= double(sign);
  return v;
}

template <int R, int SIGN>
struct Table {
  float re[R];
  float im[R];
  constexpr Table() : re(), im() {
    for (int e = 0; e < R; ++e) {
      cd v = expi(e, R, SIGN);
      re[e] = float(v.re);
      im[e] = float(v.im);
    }
  }
};

// Radix-2 butterfly constants for w = exp(SIGN 2 pi i k / R), k < R/2: the
// larger of |cos|, |sin| (with its sign) as the factor f, the other divided
// by it as the ratio r, both rounded once from double.
template <int R, int SIGN>
struct BflyTable {
  float f[R / 2];
  float r[R / 2];
  bool by_cos[R / 2];
  constexpr BflyTable() : f(), r(), by_cos() {
    for (int k = 0; k < R / 2; ++k) {
      cd w = expi(k, R, SIGN);
      const bool bc = (w.re < 0 ? -w.re : w.re) >= (w.im < 0 ? -w.im : w.im);
      by_cos[k] = bc;
      f[k] = float(bc ? w.re : w.im);
      r[k] = float(bc ? w.im / w.re : w.re / w.im);
    }
  }
};

}  // namespace ct

// x * exp(SIGN 2 pi i e / R), e a compile-time constant after unrolling.
template <int R, int SIGN>
__device__ __forceinline__ float2 twiddle_ct(float2 x, int e) {
  constexpr ct::Table<R, SIGN> tab{};
  e %= R;
  if (e == 0) return x;
  if (4 * e == R) return rot90<SIGN>(x);
  if (2 * e == R) return make_float2(-x.x, -x.y);
  if (4 * e == 3 * R) return rot90<-SIGN>(x);
  return cmul(x, make_float2(tab.re[e], tab.im[e]));
}

// ------------------------------------------------------------- DFT kernels

template <int R, int SIGN>
struct Dft;

template <int SIGN>
struct Dft<1, SIGN> {
  static __device__ __forceinline__ void run(float2*) {}
};

template <int SIGN>
struct Dft<2, SIGN> {
  static __device__ __forceinline__ void run(float2* a) {
    float2 t = a[0];
    a[0] = cadd(t, a[1]);
    a[1] = csub(t, a[1]);
  }
};

template <int SIGN>
struct Dft<3, SIGN> {
  static __device__ __forceinline__ void run(float2* a) {
    // w = exp(SIGN 2 pi i / 3) = -1/2 + SIGN i sqrt(3)/2
    constexpr float s3 = 0.86602540378443864676f;
    float2 sum = cadd(a[1], a[2]), dif = csub(a[1], a[2]);
    float2 mid = make_float2(a[0].x - 0.5f * sum.x, a[0].y - 0.5f * sum.y);
    float2 rot = rot90<SIGN>(cscale(dif, s3));
    a[0] = cadd(a[0], sum);
    a[1] = cadd(mid, rot);
    a[2] = csub(mid, rot);
  }
};

template <int SIGN>
struct Dft<4, SIGN> {
  static __device__ __forceinline__ void run(float2* a) {
    float2 a0 = cadd(a[0], a[2]), a1 = csub(a[0], a[2]);
    float2 b0 = cadd(a[1], a[3]), b1 = rot90<SIGN>(csub(a[1], a[3]));
    a[0] = cadd(a0, b0);
    a[1] = cadd(a1, b1);
    a[2] = csub(a0, b0);
    a[3] = csub(a1, b1);
  }
};

constexpr int first_factor(int r) { return r % 4 == 0 ? 4 : (r % 2 == 0 ? 2 : 3); }
constexpr bool is_pow2(int r) { return r > 0 && (r & (r - 1)) == 0; }

// Radix-2 butterfly of decimation in time with a compile-time twiddle
// w = exp(SIGN 2 pi i k / R): (e, o) -> (e + w o, e - w o).  A general w is
// factored through its larger component (Goedecker's form for
// multiply-add hardware): w o = c (o + i (s / c) o) when |c| >= |s|, else
// s ((c / s) o + i o), so the butterfly is 2 + 4 fused multiply-adds
// instead of a complex multiply (2 multiplies + 2 multiply-adds) and 4 adds.
template <int R, int SIGN>
__device__ __forceinline__ void bfly2(float2& e, float2& o, int k) {
  const float2 a = e;
  if (k == 0) {
    e = cadd(a, o);
    o = csub(a, o);
    return;
  }
  if (4 * k == R) {
    const float2 t = rot90<SIGN>(o);
    e = cadd(a, t);
    o = csub(a, t);
    return;
  }
  constexpr ct::BflyTable<R, SIGN> tab{};
  const bool by_cos = tab.by_cos[k];
  const float f = tab.f[k], r = tab.r[k];  // the factor taken out, the ratio left in
  float2 t;
  if (by_cos) t = make_float2(fmaf(-r, o.y, o.x), fmaf(r, o.x, o.y));
  else t = make_float2(fmaf(r, o.x, -o.y), fmaf(r, o.y, o.x));
  e = make_float2(fmaf(f, t.x, a.x), fmaf(f, t.y, a.y));
  o = make_float2(fmaf(-f, t.x, a.x), fmaf(-f, t.y, a.y));
}

// Power-of-two R >= 8: radix-2 decimation in time, X[k] = E[k] + w^k O[k],
// X[k + R/2] = E[k] - w^k O[k] with E, O the (R/2)-point transforms of the
// even and odd samples, recursively down to the 4-point transform.
template <int R, int SIGN>
struct DftPow2 {
  static __device__ __forceinline__ void run(float2* a) {
    constexpr int H = R / 2;
    float2 e[H], o[H];
#pragma unroll
    for (int i = 0; i < H; ++i) {
      e[i] = a[2 * i];
      o[i] = a[2 * i + 1];
    }
    DftPow2<H, SIGN>::run(e);
    DftPow2<H, SIGN>::run(o);
#pragma unroll
    for (int k = 0; k < H; ++k) {
      bfly2<R, SIGN>(e[k], o[k], k);
      a[k] = e[k];
      a[k + H] = o[k];
    }
  }
};

template <int SIGN>
struct DftPow2<4, SIGN> {
  static __device__ __forceinline__ void run(float2* a) { Dft<4, SIGN>::run(a); }
};

// Composite R = F * Q, decimation in time on n = f + F q; powers of two from
// 8 up take the radix-2 form above.
template <int R, int SIGN>
struct Dft {
  static_assert(R % 2 == 0 || R % 3 == 0, "DFT size must be a product of 2 and 3");
  static constexpr int F = first_factor(R);
  static constexpr int Q = R / F;
  static __device__ __forceinline__ void run(float2* a) {
    if constexpr (is_pow2(R) && R >= 8) {
      DftPow2<R, SIGN>::run(a);
      return;
    }
    float2 b[F][Q];
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
      for (int q = 0; q < Q; ++q) b[f][q] = a[f + F * q];
#pragma unroll
    for (int f = 0; f < F; ++f) Dft<Q, SIGN>::run(b[f]);
#pragma unroll
    for (int k = 0; k < Q; ++k) {
      float2 t[F];
#pragma unroll
      for (int f = 0; f < F; ++f) t[f] = twiddle_ct<R, SIGN>(b[f][k], f * k);
      Dft<F, SIGN>::run(t);
#pragma unroll
      for (int s = 0; s < F; ++s) a[k + Q * s] = t[s];
    }
  }
};

template <int R, int SIGN>
__device__ __forceinline__ void dft(float2* a) {
  Dft<R, SIGN>::run(a);
}

}  // namespace spectre
