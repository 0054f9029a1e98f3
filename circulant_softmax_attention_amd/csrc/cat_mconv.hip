// cat_mconv.hip -- the 1D FFT-convolution for transform length 1024 with the
// DFT stages on the matrix cores (gfx950, bf16 storage).
//
// CAT evaluates O_h = circ(z*_h) V_h as IFFT(FFT(z*_h) . FFT(V_h)) (CAT:
// Circular-Convolutional Attention for Sub-Quadratic Transformers, "Key
// designs: FFT-accelerated computation").  Two real channels c, c' form one
// complex line c + i c'; since the filter is real, one complex convolution
// gives both.  With L = 1024 = 32 x 32 each transform is two radix-32 passes,
// and a radix-32 pass over a whole line is a 32 x 32 complex matrix product:
//
//   forward,  n = 32 a + b, k = k1 + 32 k2:
//     Y[b][k1]  = sum_a x[32 a + b] F[a][k1]           (F[j][k] = w^(j k), w = e^(-2 pi i / 32))
//     Y'        = Y . W^(b k1)                          (W = e^(-2 pi i / 1024))
//     X[k2][k1] = sum_b F[k2][b] Y'[b][k1]              (X[k1 + 32 k2] of the DFT)
//   product with the filter spectrum S[k1 + 32 k2] = FFT(z*)[k]
//   inverse,  n = a + 32 b':
//     U[k1][a]  = sum_k2 P[k2][k1] conj F[k2][a]
//     U'        = U . conj W^(a k1)
//     o[b'][a]  = sum_k1 conj F[b'][k1] U'[k1][a]       (o at token a + 32 b')
//
// Each product runs as v_mfma_f32_16x16x32_f16 (fp16 operands, fp32
// accumulation): a 32 x 32 x 32 complex product is 2 x 2 output tiles, each
// four real MFMAs.  The stages chain in registers: an MFMA result holds its
// row index across the 4 lane groups (4 rows each) and its column index
// across the 16 lanes of a group, which is exactly how the next MFMA's
// operand holds its contracted index and its kept index, so each stage
// contracts the previous result's row index and no data moves between lanes.
// (K positions are paired slot by slot between the two operands, so any
// consistent slot order works; slot s of lane group g stands for index
// 4 g + (s mod 4) + 16 (s / 4), the order a result's rows come in.)
//
// Range: fp16 has 11 significand bits and a range of 6e-5 .. 65504.  Each
// line is scaled by a power of two so that its largest input part lies in
// [8, 16) (block floating point).  Twiddles and the spectrum product run as
// packed fp16 arithmetic on the operands the next product takes (the fp32
// MFMA results are converted once, then multiplied two values per
// instruction); both twiddle tables are W^(.)/32 and its conjugate, and the
// spectrum S carries no 1/L, so the 1/L of the inverse is the two 1/32.
// With N = 1024 the spectrum is made from e^(z - max) (no softmax sum): S is
// FFT(e^(z - max)) over its k = 0 term dc (the sum), split into an exact
// power of two 2^-f on the operands (2^f <= dc < 2^(f + 1), so |S| < 2) and
// the fp32 factor 2^f / dc on the outputs; with N < 1024 the softmax is
// normalised first and |S| <= 1.  Bounds (|part| <= |value|, sums of 32
// terms): pass-1 results < 32 x 16 sqrt2 < 2^10, times 1/32 < 2^5; pass-2
// results < 2^10; times S < 2^11; pass-3 results < 2^15.5 < 65504, times
// 1/32 < 2^11; the last products accumulate in fp32.  The line scale, a
// power of two, is divided out exactly at the end.

// Workgroup: one (batch, head, group of 16 channels) = 8 complex lines,
// 4 waves of 2 lines each (wave w takes channel pair w of each 8-channel
// half); three workgroups share a compute unit, so every unit gets the same
// number of lines at the headline shape.  V arrives in the blocked layout
// with 8-channel groups ([N][8] per group, 16 bytes per token), so the two
// halves are separate 16 KB runs.  They are staged into LDS by 16-byte
// LDS-DMA, the second only once the first has landed: with every
// workgroup's requests in flight at once the memory system serves them
// together, so holding the second halves back lets the first halves arrive
// at full bandwidth, and the second halves stream in under the first lines'
// transforms.  The per-lane DFT constants and twiddles come from an 8 KB
// table made on the host in double precision.  Every wave computes the
// head's softmax spectrum itself, in registers, while the first half is in
// flight (no wave waits on another for it).  Each wave reads its line's
// column and writes the line's outputs back into the same column; the block
// then leaves as 16-byte stores of the 32-byte row segments of O, and the
// groups of one head run on one XCD, so their segments meet in its L2.
#include "cat_common.hpp"
#include "cat_internal.hpp"

namespace cat {

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 half8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f2v;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 h2v;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 b2v;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned short)))) unsigned short u2v;

namespace {

constexpr int ML = 1024;      // transform length
constexpr int MCG = 16;       // channels per workgroup (8 complex lines)
constexpr int MNTHR = 256;
constexpr int GROUP_BYTES = ML * 16;  // one 8-channel group in LDS: [1024 tokens][16 bytes]

// 8 complex values in the K slots of one MFMA operand (also the layout of
// the twiddles and of the spectrum that multiply such an operand).
struct C8 {
  half8 re, im;
};
// One 16 x 16 complex result tile (4 values per lane).
struct CT {
  floatx4 re, im;
};
// A constant operand: re, im and -im of F entries.
struct K8 {
  half8 re, im, nim;
};

__device__ __forceinline__ floatx4 mm(const half8& a, const half8& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// data as the A operand (rows = its kept index), constant as B.  conj flips
// the sign of the constant's imaginary part.
template <bool CONJ>
__device__ __forceinline__ CT mul_dA(const C8& d, const K8& k) {
  const half8& ki = CONJ ? k.nim : k.im;
  const half8& kn = CONJ ? k.im : k.nim;
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  CT r;
  r.re = mm(d.im, kn, mm(d.re, k.re, z));
  r.im = mm(d.im, k.re, mm(d.re, ki, z));
  return r;
}
// constant as the A operand, data as B (columns = its kept index).
template <bool CONJ>
__device__ __forceinline__ CT mul_dB(const K8& k, const C8& d) {
  const half8& ki = CONJ ? k.nim : k.im;
  const half8& kn = CONJ ? k.im : k.nim;
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  CT r;
  r.re = mm(kn, d.im, mm(k.re, d.re, z));
  r.im = mm(ki, d.re, mm(k.re, d.im, z));
  return r;
}
// Two fp32 values to one fp16 pair (round to nearest even, one instruction).
__device__ __forceinline__ uint32_t cvt2(float x, float y) {
  const h2v h = __builtin_convertvector((f2v{x, y}), h2v);
  return __builtin_bit_cast(uint32_t, h);
}
// Two fp32 values to one bf16 pair (round to nearest even, one instruction).
__device__ __forceinline__ uint32_t cvt2bf(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v{x, y}), b2v));
}
// Operand whose slot s = v + 4 y takes value v of tile y (the two tiles
// stacked along the contracted index), converted to fp16.
__device__ __forceinline__ C8 stack(const CT& t0, const CT& t1) {
  union {
    uint32_t u[4];
    half8 h;
  } re, im;
  re.u[0] = cvt2(t0.re[0], t0.re[1]);
  re.u[1] = cvt2(t0.re[2], t0.re[3]);
  re.u[2] = cvt2(t1.re[0], t1.re[1]);
  re.u[3] = cvt2(t1.re[2], t1.re[3]);
  im.u[0] = cvt2(t0.im[0], t0.im[1]);
  im.u[1] = cvt2(t0.im[2], t0.im[3]);
  im.u[2] = cvt2(t1.im[0], t1.im[1]);
  im.u[3] = cvt2(t1.im[2], t1.im[3]);
  return C8{re.h, im.h};
}
// Slot-wise complex product d . t (CONJ: d . conj t) in packed fp16.
template <bool CONJ>
__device__ __forceinline__ C8 cmul8(const C8& d, const C8& t) {
  C8 r;
  if (!CONJ) {
    r.re = __builtin_elementwise_fma(d.re, t.re, -(d.im * t.im));
    r.im = __builtin_elementwise_fma(d.re, t.im, d.im * t.re);
  } else {
    r.re = __builtin_elementwise_fma(d.re, t.re, d.im * t.im);
    r.im = __builtin_elementwise_fma(d.im, t.re, -(d.re * t.im));
  }
  return r;
}
// Float max and sum over the wave, the same DPP pattern (a mirror swap adds
// the partner's partial, which after the quad steps holds its group's total).
template <bool SUM>
__device__ __forceinline__ float wave_reduce_f(float x) {
  auto op = [](float p, float q) { return SUM ? p + q : fmaxf(p, q); };
  auto dpp = [](float v, int ctrl) {
    const int i = __float_as_int(v);
    switch (ctrl) {
      case 0: return __int_as_float(__builtin_amdgcn_update_dpp(i, i, 0xB1, 0xF, 0xF, false));
      case 1: return __int_as_float(__builtin_amdgcn_update_dpp(i, i, 0x4E, 0xF, 0xF, false));
      case 2: return __int_as_float(__builtin_amdgcn_update_dpp(i, i, 0x141, 0xF, 0xF, false));
      default: return __int_as_float(__builtin_amdgcn_update_dpp(i, i, 0x140, 0xF, 0xF, false));
    }
  };
  x = op(x, dpp(x, 0));
  x = op(x, dpp(x, 1));
  x = op(x, dpp(x, 2));
  x = op(x, dpp(x, 3));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return op(op(r0, r1), op(r2, r3));
}
// Largest value over the wave (non-negative ints): DPP max within each row
// of 16 lanes (quad swaps, then the half-row and row mirrors), then the four
// row results.
__device__ __forceinline__ int wave_max_u(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false));  // row_mirror
  const int r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const int r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// 2^e as a float (|e| <= 126).
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }
// Power of two that brings m into [lo, 2 lo) (lo = 2^target); 1 for m == 0.
__device__ __forceinline__ int scale_exp(float m, int target) {
  if (!(m > 0.f)) return 0;
  const int e = (int)((__float_as_uint(m) >> 23) & 0xff) - 127;  // m in [2^e, 2^(e+1)) (normal m)
  int s = target - e;
  s = s < -120 ? -120 : (s > 120 ? 120 : s);
  return s;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// LDS-DMA: every lane's 16 (or 4) bytes at g land at lds + 16 (or 4) x lane.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
// Wait until at most n of this wave's vector-memory operations are in flight
// (they retire in issue order, LDS-DMA included).
template <int n>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}

// The lane's 16 logit positions in the first pass's operand (slot s of
// row block bb): position t of the length-1024 circle takes logit t (t < N),
// t - 1024 + N (t > 1024 - N; the periodic extension), or none (-1).
__device__ __forceinline__ int logit_src(int t, int N) { return t < N ? t : (t > ML - N ? t - ML + N : -1); }
__device__ __forceinline__ int logit_pos(int lo, int grp, int bb, int s) {
  return 32 * (4 * grp + (s & 3) + 16 * (s >> 2)) + lo + 16 * bb;
}

// FULL: N == 1024, no token beyond N.
template <bool FULL>
__global__ __launch_bounds__(MNTHR, 3) void mconv_kernel(ConvArgs a) {
  __shared__ __attribute__((aligned(16))) char grps[2 * GROUP_BYTES];  // the two 8-channel groups
  __shared__ __attribute__((aligned(16))) half8 ctab[8 * 64];           // the per-lane constants
  // The (b, h) filter spectrum as the operands it multiplies: [kb][part][lane]
  // holds the real (part 0) or imaginary (part 1) halves of the lane's
  // spectrum operand for column block kb.
  __shared__ __attribute__((aligned(16))) uint4 spk[2 * 2 * 64];
  __shared__ __attribute__((aligned(16))) float zlog[ML];  // the (b, h) logits
  __shared__ float dcs;  // N = 1024: the k = 0 term of the unnormalised spectrum
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lo = lane & 15, grp = lane >> 4;
  const int q = xcd_remap(blockIdx.x, gridDim.x);
  const int wgh = a.ng >> 1;  // workgroups per head
  const int bh = q / wgh, g = q - bh * wgh;
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N;
  // The half taken first alternates between neighbouring workgroups, so that
  // the first wave of requests covers both halves of the address range.
  const int first = q & 1;

  // ---- loads, in the order they are needed, by LDS-DMA: a quarter of the
  // constant table (2 KB a wave), of the logits line and of the first group
  // (4 KB a wave).  The second group is
  // requested only once the first has landed: with every workgroup's
  // requests in flight at once the memory system serves them together, so
  // holding the second groups back lets the first groups arrive at full
  // bandwidth, and the second groups stream in under the first lines'
  // transforms.
  {
    const char* tg = reinterpret_cast<const char*>(a.mtab);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = 2 * wave + i;
      lds_dma16(tg + piece * 1024 + lane * 16, __builtin_amdgcn_readfirstlane(lds_addr(ctab) + piece * 1024));
    }
  }
  {
    // The logits, 4 bytes a lane, already in the order the spectrum reads
    // them: word 4 (64 j + l) + e of zlog is the logit of slot s = (4 j + e)
    // mod 8 in row block bb = (4 j + e) / 8 of lane l's first pass operand
    // (positions with no logit take logit 0 and are masked where used).
    const float* zr = a.logits + (size_t)bh * N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = 256 * wave + 64 * i + lane;  // destination word
      const int j = 4 * (p >> 8) + (p & 3), l = (p >> 2) & 63;
      const int src = logit_src(logit_pos(l & 15, l >> 4, j >> 3, j & 7), N);
      lds_dma4(zr + (src < 0 ? 0 : src), __builtin_amdgcn_readfirstlane(lds_addr(zlog) + (256 * wave + 64 * i) * 4));
    }
  }
  // A quarter of group gi: rows 256 w .. 256 w + 255, 64 per DMA (rows at or
  // beyond N repeat row N - 1, never used).
  auto dma_group = [&](int gi) {
    const char* src = reinterpret_cast<const char*>(a.V) + ((size_t)bh * a.ng + 2 * g + gi) * (size_t)N * 16;
    const uint32_t dst = lds_addr(grps) + (uint32_t)(gi * GROUP_BYTES);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n0 = 64 * (4 * wave + i), n = n0 + lane;
      const int ns = (FULL || n < N) ? n : N - 1;
      lds_dma16(src + (size_t)ns * 16, __builtin_amdgcn_readfirstlane(dst + (uint32_t)n0 * 16));
    }
  };
  dma_group(first);

  // ---- the constants: F[lo + 16 x][4 grp + v + 16 y] (slot v + 4 y) and one
  // twiddle table for both twiddle steps: tw[x] slot v + 4 y =
  // W^((16 y + 4 grp + v)(lo + 16 x)) / 32, which is W^(b k1) / 32 for the
  // forward operand of column block k1 = lo + 16 x (b = 16 y + 4 grp + v) and,
  // conjugated, conj W^(a k1) / 32 for the inverse operand of column block
  // a = lo + 16 x (k1 = 16 y + 4 grp + v).
  wait_vm<4>();     // this wave's table and logits pieces are in LDS
  __syncthreads();  // and every other wave's
  K8 kf[2];
  C8 tw[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    kf[x].re = ctab[(2 * x) * 64 + lane];
    kf[x].im = ctab[(2 * x + 1) * 64 + lane];
    kf[x].nim = -kf[x].im;
    tw[x].re = ctab[(4 + 2 * x) * 64 + lane];
    tw[x].im = ctab[(5 + 2 * x) * 64 + lane];
  }

  {
    // ---- the filter spectrum S[k1 + 32 k2] = FFT(softmax line)[k], a
    // quarter per wave, while the first group is in flight: wave w makes the
    // 16 x 16 tile of column block kb = w mod 2 and row block k2b = w / 2 of
    // the second pass's result (the first pass only for its column block)
    // and leaves it in LDS in the layout of the operands it multiplies.  Softmax in fp32 (each
    // logit counted once in the sum: the positions t < N; every wave takes
    // the whole line's max and sum itself), then the two forward passes as
    // for the data lines, the first with a real input (two MFMAs a tile).
    const int kb = wave & 1, k2b = wave >> 1;
    float ez_[2][8];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const float4 z4 = reinterpret_cast<const float4*>(zlog)[j4 * 64 + lane];
      ez_[j4 >> 1][4 * (j4 & 1)] = z4.x;
      ez_[j4 >> 1][4 * (j4 & 1) + 1] = z4.y;
      ez_[j4 >> 1][4 * (j4 & 1) + 2] = z4.z;
      ez_[j4 >> 1][4 * (j4 & 1) + 3] = z4.w;
    }
    float mz = -INFINITY;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (!FULL && logit_src(logit_pos(lo, grp, bb, s), N) < 0) ez_[bb][s] = -INFINITY;
        mz = fmaxf(mz, ez_[bb][s]);
      }
    mz = wave_reduce_f<false>(mz);
    // e^(z - max) <= 1, times 8 (or, with N < 1024, divided by the sum over
    // t < N, the largest probability brought into [8, 16))
    float sz = 8.f;
    int ez = 3;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int s = 0; s < 8; ++s) ez_[bb][s] = __expf(ez_[bb][s] - mz);
    if (!FULL) {
      float se = 0.f;
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int s = 0; s < 8; ++s)
          if (logit_pos(lo, grp, bb, s) < N) se += ez_[bb][s];
      se = wave_reduce_f<true>(se);
      ez = scale_exp(1.f / se, 3);
      sz = pow2f(ez) / se;
    }
    const K8& k1f = kb ? kf[1] : kf[0];
    const K8& k2f = k2b ? kf[1] : kf[0];
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    CT s1t[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      half8 xr;
#pragma unroll
      for (int s = 0; s < 8; ++s) xr[s] = (_Float16)(ez_[bb][s] * sz);
      s1t[bb].re = mm(xr, k1f.re, zero);
      s1t[bb].im = mm(xr, k1f.im, zero);
    }
    const CT s2t = mul_dB<false>(k2f, cmul8<false>(stack(s1t[0], s1t[1]), kb ? tw[1] : tw[0]));
    const float unscale = pow2f(5 - ez);  // x 32 / 2^ez (N = 1024: FFT(e^(z - max)), normalised below)
    uint2 re, im;
    re.x = cvt2(s2t.re[0] * unscale, s2t.re[1] * unscale);
    re.y = cvt2(s2t.re[2] * unscale, s2t.re[3] * unscale);
    im.x = cvt2(s2t.im[0] * unscale, s2t.im[1] * unscale);
    im.y = cvt2(s2t.im[2] * unscale, s2t.im[3] * unscale);
    reinterpret_cast<uint2*>(&spk[(2 * kb) * 64 + lane])[k2b] = re;
    reinterpret_cast<uint2*>(&spk[(2 * kb + 1) * 64 + lane])[k2b] = im;
    if (FULL && wave == 0 && lane == 0) dcs = s2t.re[0] * unscale;  // k1 = 0, k2 = 0
  }

  // Every token this lane reads or writes is lo + 128 grp + off, off a
  // multiple of 16: one per-lane base and compile-time offsets.
  const uint32_t lane_row = (uint32_t)(lo + 128 * grp) * 16 + wave * 4;
  C8 sk[2];
  float cf = 1.f;  // the part of the spectrum's normalisation applied to the outputs
#pragma unroll 1
  for (int li = 0; li < 2; ++li) {
    char* const lb = grps + (li ^ first) * GROUP_BYTES + lane_row;
    wait_vm<0>();  // this wave's quarter of group li ^ first is in LDS
    __syncthreads();  // and every other wave's (and, the first time, every spectrum tile)
    if (li == 0) {
      dma_group(first ^ 1);
#pragma unroll
      for (int c = 0; c < 2; ++c)
        sk[c] = C8{__builtin_bit_cast(half8, spk[(2 * c) * 64 + lane]), __builtin_bit_cast(half8, spk[(2 * c + 1) * 64 + lane])};
      if (FULL) {
        // S = FFT(e^(z - max)) / its k = 0 term dc (the sum of e^(z - max),
        // 1 <= dc <= 1024): the operands take 2^-f (exact; |S 2^-f| < 2 with
        // 2^f <= dc < 2^(f + 1)), the output the rest, 2^f / dc, in fp32.
        const float dc = dcs;
        const int f = (int)((__float_as_uint(dc) >> 23) & 0xff) - 127;
        cf = pow2f(f) / dc;
        const _Float16 r = (_Float16)pow2f(-f);
        const half8 rh = {r, r, r, r, r, r, r, r};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          sk[c].re *= rh;
          sk[c].im *= rh;
        }
      }
    }
    // ---- input: x[32 a + b], b = lo + 16 bb, a in the slots; bf16 pairs
    uint32_t xw[2][8];
    u2v mw = {0, 0};  // largest |part| of each half as bf16 bits (monotonic in the magnitude)
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int off = 32 * ((s & 3) + 16 * (s >> 2)) + 16 * bb;  // token - lo - 128 grp
        const uint32_t w = *reinterpret_cast<const uint32_t*>(lb + off * 16);
        xw[bb][s] = (FULL || lo + 128 * grp + off < N) ? w : 0u;
        mw = __builtin_elementwise_max(mw, __builtin_bit_cast(u2v, xw[bb][s] & 0x7fff7fffu));
      }
    const int mb = max((int)mw[0], (int)mw[1]);
    const int e1 = scale_exp(__uint_as_float((uint32_t)wave_max_u(mb) << 16), 3);  // largest part -> [8, 16)
    const float s1 = pow2f(e1);
    C8 x1[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      union {
        uint32_t u[4];
        half8 h;
      } re, im;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w0 = xw[bb][2 * j], w1 = xw[bb][2 * j + 1];
        re.u[j] = cvt2(__uint_as_float(w0 << 16) * s1, __uint_as_float(w1 << 16) * s1);
        im.u[j] = cvt2(__uint_as_float(w0 & 0xffff0000u) * s1, __uint_as_float(w1 & 0xffff0000u) * s1);
      }
      x1[bb] = C8{re.h, im.h};
    }

    // ---- forward pass 1: D1[bb][kb], rows b = 16 bb + 4 grp + v, cols k1 = lo + 16 kb
    CT d1[2][2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) d1[bb][kb] = mul_dA<false>(x1[bb], kf[kb]);
    // ---- twiddle W^(b k1) / 32, then forward pass 2: D2[k2b][kb], rows k2 = 16 k2b + 4 grp + v, cols k1
    C8 y2[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) y2[kb] = cmul8<false>(stack(d1[0][kb], d1[1][kb]), tw[kb]);
    CT d2[2][2];
#pragma unroll
    for (int k2b = 0; k2b < 2; ++k2b)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) d2[k2b][kb] = mul_dB<false>(kf[k2b], y2[kb]);
    C8 p3[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) p3[kb] = stack(d2[0][kb], d2[1][kb]);

    // ---- spectrum product, then inverse pass 1: D3[kb][ab], rows k1 = 16 kb + 4 grp + v, cols a = lo + 16 ab
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) p3[kb] = cmul8<false>(p3[kb], sk[kb]);
    CT d3[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ab = 0; ab < 2; ++ab) d3[kb][ab] = mul_dA<true>(p3[kb], kf[ab]);
    // ---- twiddle conj W^(a k1) / 32, then inverse pass 2: D4[bb][ab], rows b' = 16 bb + 4 grp + v,
    //      cols a; token a + 32 b'
    C8 u4[2];
#pragma unroll
    for (int ab = 0; ab < 2; ++ab) u4[ab] = cmul8<true>(stack(d3[0][ab], d3[1][ab]), tw[ab]);
    const float inv = pow2f(-e1) * cf;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int ab = 0; ab < 2; ++ab) {
        const CT d4 = mul_dB<true>(kf[bb], u4[ab]);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int off = 16 * ab + 32 * (16 * bb + v);  // token - lo - 128 grp
          if (FULL || lo + 128 * grp + off < N)
            *reinterpret_cast<uint32_t*>(lb + off * 16) = cvt2bf(d4.re[v] * inv, d4.im[v] * inv);
        }
      }
  }
  __syncthreads();

  // ---- out: lanes 0..31 of a wave take the first 16 bytes (group 0) of
  // 32 consecutive tokens' row segments, lanes 32..63 the second 16 bytes.
  {
    char* ob = reinterpret_cast<char*>(a.O) + ((size_t)b * N * a.D + (size_t)h * a.d + (size_t)g * MCG) * 2;
    const int c = lane >> 5;
#pragma unroll 4
    for (int i = 0; i < 8; ++i) {
      const int n = 32 * (wave + 4 * i) + (lane & 31);
      if (FULL || n < N) {
        const uint4 v = *reinterpret_cast<const uint4*>(grps + c * GROUP_BYTES + n * 16);
        *reinterpret_cast<uint4*>(ob + (size_t)n * a.D * 2 + c * 16) = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_mconv(const ConvArgs& a, hipStream_t s, const LaunchTiming* t) {
  if (a.N > ML || a.N < 1 || a.d % MCG != 0 || a.ng != a.d / 8 || a.logits == nullptr || a.mtab == nullptr)
    return hipErrorInvalidValue;
  const int blocks = a.B * a.H * (a.d / MCG);
  if (a.N == ML) return launch_k(mconv_kernel<true>, dim3(blocks), dim3(MNTHR), 0, s, t, a);
  return launch_k(mconv_kernel<false>, dim3(blocks), dim3(MNTHR), 0, s, t, a);
}

}  // namespace cat
