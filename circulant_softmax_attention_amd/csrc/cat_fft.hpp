// cat_fft.hpp -- register-resident mixed-radix DFT building blocks for gfx950.
//
// The circulant product circ(w) v equals IFFT(FFT(w) . FFT(v)) (CAT:
// Circular-Convolutional Attention for Sub-Quadratic Transformers, "Key
// designs: FFT-accelerated computation"; the 2D form, a BCCB matrix times a
// vector as a 2D convolution, is in Vision Transformers are Circulant
// Attention Learners, "What does this finding overturn?").  This header holds
// the arithmetic pieces the kernels compose into those transforms:
//
//   * Dft<N, INV>::run(x): an in-place length-N DFT of N complex values held
//     in registers, natural order in and out, fully unrolled.  Forward uses
//     W = exp(-2 pi i / N); INV uses the conjugate and is NOT scaled by 1/N.
//     Composite N is split Cooley-Tukey style into radix 3, 2, 4 and 8 steps
//     whose twiddles are compile-time constants; 7 is a direct
//     symmetric-pair DFT (so 7, 14, 28 and 56 are lengths too).
//   * compile-time cos/sin of 2 pi k / n in double precision (Taylor series
//     after an exact octant reduction), rounded once to float.
//
// All indices into the register arrays are compile-time constants (sfor), so
// the arrays stay in VGPRs.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#define CAT_HD __host__ __device__ __forceinline__

namespace cat {

struct cf {
  float x, y;
};

CAT_HD cf cfm(float a, float b) {
  cf r;
  r.x = a;
  r.y = b;
  return r;
}
CAT_HD cf operator+(cf a, cf b) { return cfm(a.x + b.x, a.y + b.y); }
CAT_HD cf operator-(cf a, cf b) { return cfm(a.x - b.x, a.y - b.y); }
// a * (c + i s)
CAT_HD cf cmul(cf a, float c, float s) {
  return cfm(fmaf(a.x, c, -(a.y * s)), fmaf(a.x, s, a.y * c));
}
CAT_HD cf cmul(cf a, cf b) { return cmul(a, b.x, b.y); }
// a * conj(b)
CAT_HD cf cmulc(cf a, cf b) { return cmul(a, b.x, -b.y); }
CAT_HD cf cscale(cf a, float s) { return cfm(a.x * s, a.y * s); }

// ------------------------------------------------------------ static for
template <int B, int E, class F>
CAT_HD void sfor(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    sfor<B + 1, E>(f);
  }
}

// ------------------------------------------------------------ compile-time trig
namespace ct {
constexpr double kHalfPi = 1.57079632679489661923132169163975144;
// |x| <= pi/4: 14 Taylor terms reach below double rounding.
constexpr double sin_series(double x) {
  double x2 = x * x, term = x, sum = x;
  for (int n = 1; n < 14; ++n) {
    term *= -x2 / (double)((2 * n) * (2 * n + 1));
    sum += term;
  }
  return sum;
}
constexpr double cos_series(double x) {
  double x2 = x * x, term = 1.0, sum = 1.0;
  for (int n = 1; n < 14; ++n) {
    term *= -x2 / (double)((2 * n - 1) * (2 * n));
    sum += term;
  }
  return sum;
}
struct cs {
  double c, s;
};
// cos and sin of 2 pi k / n.  The angle is split exactly into a whole number
// of quarter turns plus (pi/2) r / n with 0 <= r < n, and the remainder is
// folded below pi/4 before the series is evaluated.
constexpr cs cossin_2pi(long k, long n) {
  k %= n;
  if (k < 0) k += n;
  const long q = (4 * k) / n;
  const long r = 4 * k - q * n;
  double c0 = 0, s0 = 0;
  if (2 * r <= n) {
    const double phi = kHalfPi * (double)r / (double)n;
    c0 = cos_series(phi);
    s0 = sin_series(phi);
  } else {
    const double psi = kHalfPi * (double)(n - r) / (double)n;
    c0 = sin_series(psi);
    s0 = cos_series(psi);
  }
  switch (q & 3) {
    case 0: return {c0, s0};
    case 1: return {-s0, c0};
    case 2: return {-c0, -s0};
    default: return {s0, -c0};
  }
}
}  // namespace ct

// x * W_N^E with W_N = exp(-2 pi i / N) (forward) or its conjugate (INV).
template <int N, bool INV, int E>
CAT_HD cf twiddle(cf a) {
  constexpr int e = ((E % N) + N) % N;
  if constexpr (e == 0) {
    return a;
  } else if constexpr (4 * e == N) {  // fwd: -i, inv: +i
    return INV ? cfm(-a.y, a.x) : cfm(a.y, -a.x);
  } else if constexpr (2 * e == N) {
    return cfm(-a.x, -a.y);
  } else if constexpr (4 * e == 3 * N) {  // fwd: +i, inv: -i
    return INV ? cfm(a.y, -a.x) : cfm(-a.y, a.x);
  } else {
    constexpr ct::cs w = ct::cossin_2pi(e, N);
    constexpr float c = (float)w.c;
    constexpr float s = INV ? (float)w.s : (float)(-w.s);
    return cmul(a, c, s);
  }
}

// ------------------------------------------------------------ DFTs
constexpr int pick_radix(int n) {
  return (n % 3 == 0) ? 3 : (n % 7 == 0 && n != 7) ? 7 : (n == 8) ? 2 : (n == 16) ? 4 : (n % 8 == 0) ? 8 : (n % 4 == 0) ? 4 : 2;
}

template <int N, bool INV>
struct Dft;

template <bool INV>
struct Dft<1, INV> {
  CAT_HD static void run(cf*) {}
};

template <bool INV>
struct Dft<2, INV> {
  CAT_HD static void run(cf* x) {
    const cf a = x[0], b = x[1];
    x[0] = a + b;
    x[1] = a - b;
  }
};

template <bool INV>
struct Dft<3, INV> {
  CAT_HD static void run(cf* x) {
    constexpr float h = 0.866025403784438646763723170752936183f;  // sin(pi/3)
    constexpr float sg = INV ? -1.0f : 1.0f;
    const cf t1 = x[1] + x[2];
    const cf d = x[1] - x[2];
    const cf t2 = cfm(fmaf(-0.5f, t1.x, x[0].x), fmaf(-0.5f, t1.y, x[0].y));
    x[0] = x[0] + t1;
    // forward: X1 = t2 - i h d, X2 = t2 + i h d; inverse swaps the signs
    x[1] = cfm(fmaf(sg * h, d.y, t2.x), fmaf(-sg * h, d.x, t2.y));
    x[2] = cfm(fmaf(-sg * h, d.y, t2.x), fmaf(sg * h, d.x, t2.y));
  }
};

// Length 7 (prime): with a_j = x[j] + x[7 - j] and b_j = x[j] - x[7 - j]
// (j = 1..3), X[0] = x[0] + sum a_j and, for k = 1..3,
//   X[k] = A_k - i B_k,  X[7 - k] = A_k + i B_k   (forward; INV swaps them)
// with A_k = x[0] + sum_j a_j cos(2 pi j k / 7), B_k = sum_j b_j sin(2 pi j k / 7).
template <bool INV>
struct Dft<7, INV> {
  CAT_HD static void run(cf* x) {
    cf a[3], b[3];
    sfor<1, 4>([&](auto J) {
      constexpr int j = decltype(J)::value;
      a[j - 1] = x[j] + x[7 - j];
      b[j - 1] = x[j] - x[7 - j];
    });
    const cf x0 = x[0];
    x[0] = x0 + a[0] + a[1] + a[2];
    sfor<1, 4>([&](auto K) {
      constexpr int k = decltype(K)::value;
      cf A = x0, Bs = cfm(0.f, 0.f);
      sfor<1, 4>([&](auto J) {
        constexpr int j = decltype(J)::value;
        constexpr ct::cs w = ct::cossin_2pi((long)j * k, 7);
        constexpr float c = (float)w.c, sn = (float)w.s;
        A = cfm(fmaf(a[j - 1].x, c, A.x), fmaf(a[j - 1].y, c, A.y));
        Bs = cfm(fmaf(b[j - 1].x, sn, Bs.x), fmaf(b[j - 1].y, sn, Bs.y));
      });
      const cf mib = cfm(Bs.y, -Bs.x);  // -i B
      x[k] = INV ? A - mib : A + mib;
      x[7 - k] = INV ? A + mib : A - mib;
    });
  }
};

template <bool INV>
struct Dft<4, INV> {
  CAT_HD static void run(cf* x) {
    const cf a = x[0] + x[2], b = x[0] - x[2], c = x[1] + x[3], d = x[1] - x[3];
    x[0] = a + c;
    x[2] = a - c;
    if constexpr (!INV) {  // X1 = b - i d, X3 = b + i d
      x[1] = cfm(b.x + d.y, b.y - d.x);
      x[3] = cfm(b.x - d.y, b.y + d.x);
    } else {
      x[1] = cfm(b.x - d.y, b.y + d.x);
      x[3] = cfm(b.x + d.y, b.y - d.x);
    }
  }
};

// Composite N = R * M.  Input index n = M n1 + n2, output index k = k1 + R k2:
//   X[k1 + R k2] = sum_{n2} W_M^{n2 k2} W_N^{n2 k1} sum_{n1} x[M n1 + n2] W_R^{n1 k1}
template <int N, bool INV>
struct Dft {
  static constexpr int R = pick_radix(N);
  static constexpr int M = N / R;
  static_assert(R * M == N && M > 1, "bad factorisation");
  CAT_HD static void run(cf* x) {
    sfor<0, M>([&](auto I2) {
      constexpr int n2 = decltype(I2)::value;
      cf t[R];
      sfor<0, R>([&](auto I1) { t[decltype(I1)::value] = x[M * decltype(I1)::value + n2]; });
      Dft<R, INV>::run(t);
      sfor<0, R>([&](auto K1) {
        constexpr int k1 = decltype(K1)::value;
        x[M * k1 + n2] = twiddle<N, INV, n2 * k1>(t[k1]);
      });
    });
    sfor<0, R>([&](auto K1) {
      constexpr int k1 = decltype(K1)::value;
      cf t[M];
      sfor<0, M>([&](auto I) { t[decltype(I)::value] = x[M * k1 + decltype(I)::value]; });
      Dft<M, INV>::run(t);
      sfor<0, M>([&](auto I) { x[M * k1 + decltype(I)::value] = t[decltype(I)::value]; });
    });
    cf y[N];
    sfor<0, R>([&](auto K1) {
      sfor<0, M>([&](auto K2) {
        y[decltype(K1)::value + R * decltype(K2)::value] = x[M * decltype(K1)::value + decltype(K2)::value];
      });
    });
    sfor<0, N>([&](auto K) { x[decltype(K)::value] = y[decltype(K)::value]; });
  }
};

constexpr int cgcd(int a, int b) { return b == 0 ? a : cgcd(b, a % b); }

// Two-pass ("four-step") decomposition of a length L1*L2 transform that the
// kernels spread over T threads per line.  Position p = L2 n1 + n2 (pass 1
// transforms over n1), spectral index k = k1 + L1 k2 (pass 2 over n2).  In
// 1D an inter-pass twiddle W_L^{n2 k1} joins the passes; on a 2D Hg x Wg grid
// (L1 = Hg, L2 = Wg, p = r Wg + c) there is none and the pair of passes is
// the 2D DFT.
//
// Each length-L1 (pass 1) or length-L2 (pass 2) DFT is held by S threads
// (S = 1 or 2): thread h of the S holds the indices congruent to h mod S, in
// and out (an even/odd split joined by one exchange between the two threads).
// With TC = T / S thread groups and t = S c + h:
//   pass 1: group c holds J1 = E S / L1 columns n2 = c + TC j; register
//           j (L1/S) + m holds n1 (in) or k1 (out) = S m + h
//   pass 2: group c holds J2 = E S / L2 rows    k1 = c + TC j; register
//           j (L2/S) + m holds n2 (in) or k2 (out) = S m + h
template <int L1_, int L2_, int S_ = 1>
struct Grid2 {
  static constexpr int L1 = L1_, L2 = L2_, L = L1_ * L2_, S = S_;
  static constexpr int T = S_ * cgcd(L1_, L2_);
  static constexpr int E = L / T;
  static constexpr int Q1 = L1_ / S_, Q2 = L2_ / S_;  // values of one DFT per thread
  static constexpr int J1 = E / Q1;
  static constexpr int J2 = E / Q2;
  static constexpr int TC = T / S_;
  static_assert(S_ == 1 || (S_ == 2 && Q1 % 2 == 0 && Q2 % 2 == 0), "split DFTs need even halves");
  // LDS row pitch (complex) of the [L1][L2] exchange tile, padded so that a
  // wave's 64-bit accesses spread over the banks.
  static constexpr int P2 = L2_ + ((L2_ % 2 == 0) ? 1 : 0);
  static constexpr int base_line = L1_ * P2;
  // line pitch = base rounded up to 2 (mod 16) complex elements
  static constexpr int LP = base_line + ((2 - base_line % 16) + 16) % 16;
};

}  // namespace cat
