// cat_score96.hip -- 2D score partials on the 96 x 96 patch grid (gfx950).
//
// Vision Transformers are Circulant Attention Learners ("Circulant Attention:
// attention rebuilt with the FFT") scores a head by the circular
// cross-correlation of Q and K on the patch grid, summed over the head's
// channels; its spectrum is sum_c FFT2(q_c) conj(FFT2(k_c)).  Two real
// channels ride in one complex line (q_c + i q_c'), and the real part of the
// inverse transform of FFT2(q pair) conj(FFT2(k pair)) is the sum of the two
// channels' correlations.  This kernel forms, for each (batch, head) and
// group of channel pairs, partial[bh][grp][k1 + 96 k2] = the sum over the
// group's pairs of that product, the same partials the generic score kernel
// writes, for the 96 x 96 grid of a 1536-pixel image at patch 16.
//
// A 96-point DFT runs on four lanes (h = h0 + 2 h1, h0 = lane bit 4, h1 =
// lane bit 5) that each hold 24 samples x[4 m + h]: a 24-point DFT in
// registers, then two radix-2 steps across the lanes, each a 2 x 2 exchange
// of register pairs between lanes 32 apart (h1) and 16 apart (h0) with the
// permlane swaps of gfx950, which move both halves of the pair in one
// instruction.  Lane (c, h) ends with X[k] for k = KB[r] + 12 h1 + KD[r] h0
// in register r.  A line is a 96 x 96 grid: pass 1 transforms the columns
// (lanes of one wave own 16 columns), an LDS exchange turns them into rows,
// pass 2 transforms the rows.  The row pitch of 98 complex values keeps both
// sides of the exchange free of bank conflicts: a half-wave writes two rows
// 8 or 24 apart (8 x 98 = 16 mod 32 float2 slots) and reads 16 consecutive
// rows at two adjacent columns (2 slots per row).
//
// Workgroup: 384 threads (96 columns x 4 lanes), one (batch, head, pair
// group); the q line and the k line of a pair go through the one 75 KB
// exchange tile in turn, so two workgroups share a CU (three waves per
// SIMD).  The q spectrum waits in registers for the k spectrum; the product
// is summed over the group's pairs in registers and stored once.
#include "cat_common.hpp"
#include "cat_fft.hpp"
#include "cat_internal.hpp"

namespace cat {
namespace {

constexpr int GS = 96;           // grid side
constexpr int NPOS = GS * GS;    // positions of one grid
constexpr int PITCH = 98;        // LDS row pitch, complex values
constexpr int NTHR = 4 * GS;     // threads per workgroup
constexpr int NR = 24;           // complex values per thread

// Second-step register pairs (r, r'): after the first step register r
// holds index g(r) = r (r < 12) or r + 12 (r >= 12) (+ 12 h1); each pair's
// indices differ by 8 or 24, so that the two rows a half-wave writes are
// 8 (mod 16) apart.
constexpr int PA[12] = {0, 1, 2, 3, 4, 5, 6, 7, 12, 13, 14, 15};
constexpr int PB[12] = {8, 9, 10, 11, 16, 17, 18, 19, 20, 21, 22, 23};
constexpr int gidx(int r) { return r < 12 ? r : r + 12; }
// Output index of register r: KB[r] + 12 h1 + KD[r] h0.
constexpr int KB[NR] = {0, 1, 2, 3, 4, 5, 6, 7, 48, 49, 50, 51, 24, 25, 26, 27, 52, 53, 54, 55, 72, 73, 74, 75};
constexpr int KD[NR] = {8, 8, 8, 8, 24, 24, 24, 24, 8, 8, 8, 8, 8, 8, 8, 8, 24, 24, 24, 24, 8, 8, 8, 8};

// 2 x 2 exchange of a complex register pair with the partner lane 16 (h0)
// or 32 (h1) away: the lower lane keeps a and receives the partner's a in b;
// the upper lane keeps b and receives the partner's b in a.
template <bool L32>
__device__ __forceinline__ void xswap(cf& a, cf& b) {
  const auto sx = L32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(a.x), __float_as_uint(b.x), false, false)
                      : __builtin_amdgcn_permlane16_swap(__float_as_uint(a.x), __float_as_uint(b.x), false, false);
  const auto sy = L32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(a.y), __float_as_uint(b.y), false, false)
                      : __builtin_amdgcn_permlane16_swap(__float_as_uint(a.y), __float_as_uint(b.y), false, false);
  a = cfm(__uint_as_float(sx[0]), __uint_as_float(sy[0]));
  b = cfm(__uint_as_float(sx[1]), __uint_as_float(sy[1]));
}

struct LaneTw {
  bool h1;
  cf w8, w24;  // W_96^(12 h1 + 8 h0), W_96^(12 h1 + 24 h0)
};

// Forward 96-point DFT over the four lanes of a column (or row): register m
// holds x[4 m + h] on entry and X[KB[m] + 12 h1 + KD[m] h0] on exit.
__device__ __forceinline__ void dft96(cf* x, const LaneTw& lt) {
  Dft<NR, false>::run(x);  // F_h[k], k = 0..23: the DFT of the lane's samples
  // Step 1, lanes 32 apart: the 48-point DFTs G_h0 of x[2 n + h0].  After the
  // exchange lane h1 holds a = F_lo[k], b = F_hi[k] with k = r + 12 h1;
  // G[k] = a + W_48^k b, G[k + 24] = a - W_48^k b, W_48^12 = -i.
  sfor<0, 12>([&](auto I) {
    constexpr int r = decltype(I)::value;
    xswap<true>(x[r], x[r + 12]);
    cf b = x[r + 12];
    b = lt.h1 ? cfm(b.y, -b.x) : b;
    b = twiddle<48, false, r>(b);
    const cf a = x[r];
    x[r] = a + b;
    x[r + 12] = a - b;
  });
  // Step 2, lanes 16 apart: X[k] = G_0[k] + W_96^k G_1[k], X[k + 48] =
  // G_0[k] - W_96^k G_1[k], with k = g(r) + 12 h1 + (g(r') - g(r)) h0.
  sfor<0, 12>([&](auto I) {
    constexpr int i = decltype(I)::value;
    constexpr int ra = PA[i], rb = PB[i];
    constexpr bool d8 = gidx(rb) - gidx(ra) == 8;
    xswap<false>(x[ra], x[rb]);
    cf b = cmul(x[rb], d8 ? lt.w8 : lt.w24);
    b = twiddle<96, false, gidx(ra)>(b);
    const cf a = x[ra];
    x[ra] = a + b;
    x[rb] = a - b;
  });
}

// NP pairs per workgroup (2; 1 for the last group of an odd pair count):
// groups grp0 .. grp0 + ngl - 1 of every (batch, head); tile is the
// workgroup's [96][PITCH] exchange tile in LDS.
template <int NP>
__device__ __forceinline__ void score96_body(const ScoreArgs& a, int grp0, int ngl, float2* tile) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h0 = (lane >> 4) & 1, h1 = lane >> 5, h = h0 + 2 * h1;
  const int col = 16 * wave + (lane & 15);  // pass-1 column, pass-2 row
  const int q = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = q / ngl, grp = grp0 + (q - bh * ngl);

  LaneTw lt;
  lt.h1 = h1 != 0;
  {
    constexpr ct::cs c8 = ct::cossin_2pi(8, GS), c12 = ct::cossin_2pi(12, GS), c20 = ct::cossin_2pi(20, GS);
    constexpr ct::cs c24 = ct::cossin_2pi(24, GS), c36 = ct::cossin_2pi(36, GS);
    // forward twiddles W^e = cos - i sin
    const cf w12 = cfm((float)c12.c, (float)-c12.s);
    lt.w8 = h0 ? (h1 ? cfm((float)c20.c, (float)-c20.s) : cfm((float)c8.c, (float)-c8.s)) : (h1 ? w12 : cfm(1.f, 0.f));
    lt.w24 = h0 ? (h1 ? cfm((float)c36.c, (float)-c36.s) : cfm((float)c24.c, (float)-c24.s)) : (h1 ? w12 : cfm(1.f, 0.f));
  }
  float2* wbase8 = tile + (12 * h1 + 8 * h0) * PITCH + col;
  float2* wbase24 = tile + (12 * h1 + 24 * h0) * PITCH + col;
  const float2* rbase = tile + col * PITCH + h;
  const int lo = h * GS + col;  // sample m of the lane: position lo + 4 m GS

  auto load = [&](const float2* __restrict__ src, cf* x) {
    sfor<0, NR>([&](auto M) {
      constexpr int m = decltype(M)::value;
      const float2 v = src[lo + 4 * m * GS];
      x[m] = cfm(v.x, v.y);
    });
  };
  // pass 1 (columns) and the exchange: x <- the grid's column spectra, by rows
  auto pass1 = [&](cf* x) {
    dft96(x, lt);
    __syncthreads();  // every lane has read the previous grid's rows
    sfor<0, NR>([&](auto R) {
      constexpr int r = decltype(R)::value;
      float2* p = (KD[r] == 8 ? wbase8 : wbase24) + KB[r] * PITCH;
      *p = make_float2(x[r].x, x[r].y);
    });
    __syncthreads();
    sfor<0, NR>([&](auto M) {
      constexpr int m = decltype(M)::value;
      const float2 v = rbase[4 * m];
      x[m] = cfm(v.x, v.y);
    });
  };

  // one pair: the q grid's spectrum waits in qs for the k grid's in ks.  The
  // scheduling fences keep each transform's temporaries to itself: loads
  // issued early or two transforms interleaved would need registers the
  // three 24-value sets (q spectrum, k grid, running sum) already take.
  cf acc[NR], qs[NR], ks[NR];
  sfor<0, NP>([&](auto P) {
    constexpr int k = decltype(P)::value;
    const size_t line = ((size_t)bh * a.npair + grp * 2 + k) * (size_t)NPOS;
    __builtin_amdgcn_sched_barrier(0);
    load(reinterpret_cast<const float2*>(a.Q) + line, qs);
    pass1(qs);
    dft96(qs, lt);  // pass 2 (rows): the q spectrum
    __builtin_amdgcn_sched_barrier(0);
    load(reinterpret_cast<const float2*>(a.K) + line, ks);
    pass1(ks);
    dft96(ks, lt);
    sfor<0, NR>([&](auto R) {
      constexpr int r = decltype(R)::value;
      acc[r] = k == 0 ? cmulc(qs[r], ks[r]) : acc[r] + cmulc(qs[r], ks[r]);
    });
  });
  // register r holds k1 = col, k2 = KB[r] + 12 h1 + KD[r] h0
  float2* dst = a.partial + ((size_t)bh * a.ngrp + grp) * NPOS + col + GS * 12 * h1;
  sfor<0, NR>([&](auto R) {
    constexpr int r = decltype(R)::value;
    dst[GS * (KB[r] + KD[r] * h0)] = make_float2(acc[r].x, acc[r].y);
  });
}

// Three waves per SIMD (two workgroups per CU) leave 168 registers a lane:
// the q spectrum, the k grid and the running sum take 144 of them.
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(3, 3))) void score96_kernel(ScoreArgs a, int grp0,
                                                                                                 int ngl) {
  extern __shared__ __attribute__((aligned(16))) float2 tile[];
  score96_body<2>(a, grp0, ngl, tile);
}
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(3, 3))) void score96_one_kernel(ScoreArgs a,
                                                                                                     int grp0, int ngl) {
  extern __shared__ __attribute__((aligned(16))) float2 tile[];
  score96_body<1>(a, grp0, ngl, tile);
}


// ------------------------------------------------------------ softmax spectrum
// The filter spectrum of one (batch, head) from its summed score spectrum,
// on the 96 x 96 grid: the scores are a = Re IFFT2(S) / sqrt(d) (S the sum
// of a.ngrp partials), a* = softmax over the grid, and the spectrum is
// FFT2(a*) / 9216 -- the same quantities the generic spectrum kernel forms
// in its scores mode.  The inverse transform runs the forward 96-point DFTs
// on conj(S): the result is conj of the inverse, whose real part is the
// same.  Workgroup: one (batch, head), the lanes of the score kernel, the
// grid through the exchange tile four times (inverse, and forward in both
// directions), block reductions for the softmax through LDS.
__global__ __launch_bounds__(NTHR) void spec96_kernel(SpecArgs a) {
  extern __shared__ __attribute__((aligned(16))) float2 tile[];  // [96][PITCH], then 8 floats
  float* red = reinterpret_cast<float*>(tile + GS * PITCH);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h0 = (lane >> 4) & 1, h1 = lane >> 5, h = h0 + 2 * h1;
  const int col = 16 * wave + (lane & 15);
  const int bh = blockIdx.x;

  LaneTw lt;
  lt.h1 = h1 != 0;
  {
    constexpr ct::cs c8 = ct::cossin_2pi(8, GS), c12 = ct::cossin_2pi(12, GS), c20 = ct::cossin_2pi(20, GS);
    constexpr ct::cs c24 = ct::cossin_2pi(24, GS), c36 = ct::cossin_2pi(36, GS);
    const cf w12 = cfm((float)c12.c, (float)-c12.s);
    lt.w8 = h0 ? (h1 ? cfm((float)c20.c, (float)-c20.s) : cfm((float)c8.c, (float)-c8.s)) : (h1 ? w12 : cfm(1.f, 0.f));
    lt.w24 = h0 ? (h1 ? cfm((float)c36.c, (float)-c36.s) : cfm((float)c24.c, (float)-c24.s)) : (h1 ? w12 : cfm(1.f, 0.f));
  }
  float2* wbase8 = tile + (12 * h1 + 8 * h0) * PITCH + col;
  float2* wbase24 = tile + (12 * h1 + 24 * h0) * PITCH + col;
  const float2* rbase = tile + col * PITCH + h;
  // register r of a transform's output <-> index KB[r] + 12 h1 + KD[r] h0 along
  // its axis; the lane's column (or row) is col
  auto exchange = [&](cf* x) {
    __syncthreads();  // every lane is done with the tile
    sfor<0, NR>([&](auto R) {
      constexpr int r = decltype(R)::value;
      float2* q = (KD[r] == 8 ? wbase8 : wbase24) + KB[r] * PITCH;
      *q = make_float2(x[r].x, x[r].y);
    });
    __syncthreads();
    sfor<0, NR>([&](auto M) {
      constexpr int m = decltype(M)::value;
      const float2 v = rbase[4 * m];
      x[m] = cfm(v.x, v.y);
    });
  };
  auto block_reduce = [&](float v, bool is_max) {
    for (int o = 32; o > 0; o >>= 1) {
      const float u = __shfl_xor(v, o);
      v = is_max ? fmaxf(v, u) : v + u;
    }
    __syncthreads();  // red is free
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < NTHR / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
    return r;
  };

  // S[k1 = col][k2 = 4 m + h], conjugated
  cf x[NR];
  sfor<0, NR>([&](auto M) { x[decltype(M)::value] = cfm(0.f, 0.f); });
  for (int g = 0; g < a.ngrp; ++g) {
    const float2* src = a.partial + ((size_t)bh * a.ngrp + g) * NPOS + col + GS * h;
    sfor<0, NR>([&](auto M) {
      constexpr int m = decltype(M)::value;
      const float2 v = src[4 * m * GS];
      x[m] = x[m] + cfm(v.x, v.y);
    });
  }
  sfor<0, NR>([&](auto M) { x[decltype(M)::value].y = -x[decltype(M)::value].y; });
  dft96(x, lt);  // over k2: row k1 = col, register r -> n2
  exchange(x);   // row n2 = col, register m -> k1 = 4 m + h
  dft96(x, lt);  // over k1: register r -> n1, column n2 = col

  // scores and their softmax over the grid
  const float ls = a.scale / (float)NPOS;
  float v[NR];
  float mx = -INFINITY;
  sfor<0, NR>([&](auto R) {
    constexpr int r = decltype(R)::value;
    v[r] = x[r].x * ls;
    mx = fmaxf(mx, v[r]);
  });
  mx = block_reduce(mx, true);
  float sum = 0.f;
  sfor<0, NR>([&](auto R) {
    constexpr int r = decltype(R)::value;
    v[r] = expf(v[r] - mx);
    sum += v[r];
  });
  sum = block_reduce(sum, false);
  const float inv_s = 1.0f / sum;
  if (a.probs != nullptr) {
    // position n1 96 + n2, n1 = KB[r] + 12 h1 + KD[r] h0, n2 = col
    float* pb = a.probs + (size_t)bh * NPOS + col + GS * 12 * h1;
    sfor<0, NR>([&](auto R) {
      constexpr int r = decltype(R)::value;
      pb[GS * (KB[r] + KD[r] * h0)] = v[r] * inv_s;
    });
  }
  // FFT2(a*) / 9216: a*[n1][n2] sits at row n1 = index of r, column n2 = col
  const float sc = inv_s / (float)NPOS;
  sfor<0, NR>([&](auto R) { x[decltype(R)::value] = cfm(v[decltype(R)::value] * sc, 0.f); });
  exchange(x);   // row n1 = col, register m -> n2 = 4 m + h
  dft96(x, lt);  // over n2: register r -> k2
  exchange(x);   // row k2 = col, register m -> n1 = 4 m + h
  dft96(x, lt);  // over n1: register r -> k1, k2 = col
  float2* dst = a.spec + (size_t)bh * NPOS;
  sfor<0, NR>([&](auto R) {
    constexpr int r = decltype(R)::value;
    const int k1 = KB[r] + 12 * h1 + KD[r] * h0;
    dst[a.transpose ? col + GS * k1 : k1 + GS * col] = make_float2(x[r].x, x[r].y);
  });
}

}  // namespace

size_t score96_lds_bytes() { return (size_t)GS * PITCH * sizeof(float2); }

hipError_t launch_spec96(const SpecArgs& a, hipStream_t s, const LaunchTiming* t) {
  if (a.N != NPOS || a.partial == nullptr || a.ngrp < 1 || a.BH < 1) return hipErrorInvalidValue;
  return launch_k(spec96_kernel, dim3((unsigned)a.BH), dim3(NTHR), score96_lds_bytes() + 8 * sizeof(float), s, t, a);
}

hipError_t launch_score96(const ScoreArgs& a, hipStream_t s, const LaunchTiming* t) {
  if (a.N != NPOS || a.et != ET_F32 || a.cg != 2 || a.ppg != 2 || a.BH < 1 || a.npair < 1 ||
      a.ngrp != (a.npair + 1) / 2)
    return hipErrorInvalidValue;
  if ((size_t)a.BH * a.ngrp > 0x7fffffffu) return hipErrorInvalidValue;
  const int full = a.npair / 2;  // groups of two pairs
  // timing: the first launch stamps the start, the last the end
  const LaunchTiming t1 = {t ? t->start : nullptr, (t && full == a.ngrp) ? t->stop : nullptr};
  const LaunchTiming t2 = {(t && full == 0) ? t->start : nullptr, t ? t->stop : nullptr};
  hipError_t e = hipSuccess;
  if (full > 0)
    e = launch_k(score96_kernel, dim3((unsigned)(a.BH * full)), dim3(NTHR), score96_lds_bytes(), s,
                 t ? &t1 : nullptr, a, 0, full);
  if (e == hipSuccess && full < a.ngrp)  // an odd pair count: the last group holds one pair
    e = launch_k(score96_one_kernel, dim3((unsigned)a.BH), dim3(NTHR), score96_lds_bytes(), s, t ? &t2 : nullptr,
                 a, full, 1);
  return e;
}

}  // namespace cat
