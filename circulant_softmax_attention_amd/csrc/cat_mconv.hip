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
//   product with the filter spectrum S[k1 + 32 k2] (1/L folded in)
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
// [8, 16) (block floating point); the first twiddle table carries 2^5 and
// the second 2^-5.  Bounds (|part| <= |value|, sums of 32 terms): pass-1
// operands < 32 x 16 sqrt2 x 2^5 < 2^15; the spectrum has |S| <= 1/L (the
// softmax sums to one and 1/L is folded in), so the inverse operands stay
// below 2^10 x sqrt2; the last products accumulate in fp32.  The line scale,
// a power of two, is divided out exactly at the end.
//
// Workgroup: one (batch, head, group of 16 channels) = 8 complex lines,
// 4 waves of 2 lines each; three workgroups share a compute unit, so every
// unit gets the same number of lines at the headline shape.  The group's
// [N][16] block of V (blocked layout, 32 bytes per token) is staged into LDS
// by 16-byte LDS-DMA (the two chunks of a row swapped by bit 3 of the token).
// Each wave reads its line's column and writes the line's outputs back into
// the same column (no other wave reads it).  The block then leaves as
// 16-byte stores of the 32-byte row segments of O; the groups of one head run
// on one XCD, so their segments meet in its L2.
#include "cat_common.hpp"
#include "cat_internal.hpp"

namespace cat {

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 half8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

namespace {

constexpr int ML = 1024;      // transform length
constexpr int MCG = 16;         // channels per workgroup (8 complex lines)
constexpr int MROWB = MCG * 2;  // bytes per token row of the V block and of the LDS tile
constexpr int TILE = ML * MROWB;
constexpr int MNTHR = 256;

// 8 complex values in the K slots of one MFMA operand.
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
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f2v;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 h2v;
__device__ __forceinline__ uint32_t cvt2(float x, float y) {
  const h2v h = __builtin_convertvector((f2v{x, y}), h2v);
  return __builtin_bit_cast(uint32_t, h);
}
// Operand whose slot s = v + 4 y takes value v of tile y (the two tiles
// stacked along the contracted index).
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
__device__ __forceinline__ float2 cmulf(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
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

// The block lives in one LDS tile [1024][32 bytes]; the 16-byte chunk j of
// token n's row sits at position j ^ bit 3 of n.
__device__ __forceinline__ uint32_t tsw(int n) { return ((uint32_t)n >> 3) & 1; }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// FULL: N == 1024, no token beyond N.
template <bool FULL>
__global__ __launch_bounds__(MNTHR) void mconv_kernel(ConvArgs a) {
  __shared__ __attribute__((aligned(16))) char blk[TILE];
  __shared__ __attribute__((aligned(16))) float2 sp[ML];  // the (b, h) filter spectrum
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lo = lane & 15, grp = lane >> 4;
  const int q = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = q / a.ng, g = q - bh * a.ng;
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N;

  // Constant operands F[lo + 16 x][4 grp + v + 16 y] (slot v + 4 y) and the
  // lane's twiddles, which are the same for all its lines, come from the
  // hardware sine and cosine (their argument is in revolutions, and every
  // angle here is an exact multiple of 1/1024 revolution):
  //   t1[bb][kb][v] = W^(b k1) x 32,      b = 16 bb + 4 grp + v, k1 = lo + 16 kb
  //   t2[kb][ab][v] = conj W^(a k1) / 32, k1 = 16 kb + 4 grp + v, a = lo + 16 ab
  K8 kf[2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int j = lo + 16 * x, k = 4 * grp + (s & 3) + 16 * (s >> 2);
      const float rev = (float)((j * k) & 31) * (1.f / 32.f);
      const float c = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
      kf[x].re[s] = (_Float16)c;
      kf[x].im[s] = (_Float16)(-sn);
      kf[x].nim[s] = (_Float16)sn;
    }
  float2 t1[2][2][4], t2[2][2][4];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int e1 = ((16 * x + 4 * grp + v) * (lo + 16 * y)) & (ML - 1);
        const float r1 = (float)e1 * (1.f / ML);
        t1[x][y][v] = make_float2(32.f * __builtin_amdgcn_cosf(r1), -32.f * __builtin_amdgcn_sinf(r1));
        t2[x][y][v] = make_float2(__builtin_amdgcn_cosf(r1) * (1.f / 32.f), __builtin_amdgcn_sinf(r1) * (1.f / 32.f));
      }
  // With logits given, wave 0 computes the filter spectrum itself, from the
  // 16 logits its lanes hold in the first pass's operand: position t of the
  // length-1024 circle takes logit t (t < N), t - 1024 + N (t > 1024 - N;
  // the periodic extension), or none.
  const bool fused = a.logits != nullptr;
  float zl[2][8];
  if (fused && wave == 0) {
    const float* zr = a.logits + (size_t)bh * N;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int t = 32 * (4 * grp + (s & 3) + 16 * (s >> 2)) + lo + 16 * bb;
        const int src = t < N ? t : (t > ML - N ? t - ML + N : -1);
        zl[bb][s] = src >= 0 ? zr[src] : -INFINITY;
      }
  }

  // The [N][16] block: 32 DMAs of 32 rows, 8 per wave; lane l fills
  // position l % 2 of row n0 + l / 2 with the global chunk (l % 2) ^ bit 3
  // of n.  Rows at or beyond N repeat row N - 1 (never used).
  const char* vblk = reinterpret_cast<const char*>(a.V) + ((size_t)bh * a.ng + g) * (size_t)N * MROWB;
  auto dma_tile = [&]() {
    const uint32_t base = lds_addr(blk);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n0 = (wave * 8 + i) * 32;
      const int n = n0 + (lane >> 1);
      const int c = (lane & 1) ^ (int)tsw(n);
      const int ns = n < N ? n : N - 1;
      lds_dma16(vblk + (size_t)ns * MROWB + c * 16, base + (uint32_t)n0 * MROWB);
    }
  };
  if (!fused) {  // the spectrum: 8 KB, two 1 KB pieces per wave
    const char* sg = reinterpret_cast<const char*>(a.spec + (size_t)bh * ML);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = wave * 2 + i;
      lds_dma16(sg + piece * 1024 + lane * 16, lds_addr(sp) + piece * 1024);
    }
  }
  dma_tile();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // the block (and the spectrum, if given) is in LDS

  // The filter spectrum S[k1 + 32 k2] = FFT(softmax line)[k] / L: softmax in
  // fp32 (each logit counted once in the sum: the positions t < N), then the
  // two forward passes as for the data lines.
  if (fused && wave == 0) {
    float mz = -INFINITY;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int s = 0; s < 8; ++s) mz = fmaxf(mz, zl[bb][s]);
    mz = wave_reduce_f<false>(mz);
    float se = 0.f;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int t = 32 * (4 * grp + (s & 3) + 16 * (s >> 2)) + lo + 16 * bb;
        zl[bb][s] = __expf(zl[bb][s] - mz);
        if (t < N) se += zl[bb][s];
      }
    se = wave_reduce_f<true>(se);
    const int ez = scale_exp(1.f / se, 3);  // largest probability 1 / se -> [8, 16)
    const float sz = pow2f(ez) / se;
    C8 x1[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        x1[bb].re[s] = (_Float16)(zl[bb][s] * sz);
        x1[bb].im[s] = (_Float16)0.f;
      }
    CT d1[2][2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        d1[bb][kb] = mul_dA<false>(x1[bb], kf[kb]);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float2 r = cmulf(make_float2(d1[bb][kb].re[v], d1[bb][kb].im[v]), t1[bb][kb][v]);
          d1[bb][kb].re[v] = r.x;
          d1[bb][kb].im[v] = r.y;
        }
      }
    const float unscale = pow2f(-ez - 15);  // / (2^ez x 32 x L)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const C8 y2 = stack(d1[0][kb], d1[1][kb]);
#pragma unroll
      for (int k2b = 0; k2b < 2; ++k2b) {
        const CT d2 = mul_dB<false>(kf[k2b], y2);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int k2 = 16 * k2b + 4 * grp + v, k1 = lo + 16 * kb;
          sp[k1 + 32 * k2] = make_float2(d2.re[v] * unscale, d2.im[v] * unscale);
        }
      }
    }
  }

  // Every token this lane reads or writes is lo + 128 grp + (a multiple of
  // 16), so bit 3 of the token, which sets the chunk position, is that of
  // lo: one per-lane base, and compile-time offsets for the rest.
  const uint32_t lane_row = (uint32_t)(lo + 128 * grp) * MROWB;
#pragma unroll 1
  for (int li = 0; li < 2; ++li) {
    const int pp = 2 * wave + li;  // channel pair (complex line) of the group
    const char* lb = blk + lane_row + ((((uint32_t)pp >> 2) ^ tsw(lo)) << 4) + (((uint32_t)pp & 3) << 2);
    // ---- input: x[32 a + b], b = lo + 16 bb, a in the slots; bf16 pairs
    uint32_t xw[2][8];
    int mb = 0;  // largest |part| as bf16 bits (monotonic in the magnitude)
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int off = 32 * ((s & 3) + 16 * (s >> 2)) + 16 * bb;  // token - lo - 128 grp
        const uint32_t w = *reinterpret_cast<const uint32_t*>(lb + off * MROWB);
        xw[bb][s] = (FULL || lo + 128 * grp + off < N) ? w : 0u;
        mb = max(mb, (int)max(xw[bb][s] & 0x7fffu, (xw[bb][s] >> 16) & 0x7fffu));
      }
    const int e1 = scale_exp(__uint_as_float((uint32_t)wave_max_u(mb) << 16), 3);  // largest part -> [8, 16)
    const float s1 = pow2f(e1);
    C8 x1[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        x1[bb].re[s] = (_Float16)(__uint_as_float(xw[bb][s] << 16) * s1);
        x1[bb].im[s] = (_Float16)(__uint_as_float(xw[bb][s] & 0xffff0000u) * s1);
      }

    // ---- forward pass 1: D1[bb][kb], rows b = 16 bb + 4 grp + v, cols k1 = lo + 16 kb
    CT d1[2][2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) d1[bb][kb] = mul_dA<false>(x1[bb], kf[kb]);
    // twiddle W^(b k1) x 2^5
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float2 r = cmulf(make_float2(d1[bb][kb].re[v], d1[bb][kb].im[v]), t1[bb][kb][v]);
          d1[bb][kb].re[v] = r.x;
          d1[bb][kb].im[v] = r.y;
        }
    // ---- forward pass 2: D2[k2b][kb], rows k2 = 16 k2b + 4 grp + v, cols k1
    C8 y2[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) y2[kb] = stack(d1[0][kb], d1[1][kb]);
    CT d2[2][2];
#pragma unroll
    for (int k2b = 0; k2b < 2; ++k2b)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) d2[k2b][kb] = mul_dB<false>(kf[k2b], y2[kb]);
    if (fused && li == 0) __syncthreads();  // wave 0's spectrum is in LDS
    // ---- spectrum product
#pragma unroll
    for (int k2b = 0; k2b < 2; ++k2b)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int k2 = 16 * k2b + 4 * grp + v, k1 = lo + 16 * kb;
          const float2 r = cmulf(make_float2(d2[k2b][kb].re[v], d2[k2b][kb].im[v]), sp[k1 + 32 * k2]);
          d2[k2b][kb].re[v] = r.x;
          d2[k2b][kb].im[v] = r.y;
        }
    // ---- inverse pass 1: D3[kb][ab], rows k1 = 16 kb + 4 grp + v, cols a = lo + 16 ab
    C8 p3[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) p3[kb] = stack(d2[0][kb], d2[1][kb]);
    CT d3[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ab = 0; ab < 2; ++ab) d3[kb][ab] = mul_dA<true>(p3[kb], kf[ab]);
    // twiddle conj W^(a k1) x 2^-5
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ab = 0; ab < 2; ++ab)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float2 r = cmulf(make_float2(d3[kb][ab].re[v], d3[kb][ab].im[v]), t2[kb][ab][v]);
          d3[kb][ab].re[v] = r.x;
          d3[kb][ab].im[v] = r.y;
        }
    // ---- inverse pass 2: D4[bb][ab], rows b' = 16 bb + 4 grp + v, cols a; token a + 32 b'
    C8 u4[2];
#pragma unroll
    for (int ab = 0; ab < 2; ++ab) u4[ab] = stack(d3[0][ab], d3[1][ab]);
    const float inv = pow2f(-e1);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int ab = 0; ab < 2; ++ab) {
        const CT d4 = mul_dB<true>(kf[bb], u4[ab]);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int off = 16 * ab + 32 * (16 * bb + v);  // token - lo - 128 grp
          if (FULL || lo + 128 * grp + off < N)
            *reinterpret_cast<uint32_t*>(const_cast<char*>(lb) + off * MROWB) = pack_bf16x2(d4.re[v] * inv, d4.im[v] * inv);
        }
      }
  }
  __syncthreads();

  // ---- out: row n of the block -> O[b][n][h d + 32 g ..], 16-byte chunks
  {
    char* ob = reinterpret_cast<char*>(a.O) + ((size_t)b * N * a.D + (size_t)h * a.d + (size_t)g * MCG) * 2;
#pragma unroll 4
    for (int i = 0; i < 8; ++i) {
      const int qq = tid + MNTHR * i;
      const int n = qq >> 1, c = qq & 1;  // global chunk c of row n
      if (n < N) {
        const uint4 v = *reinterpret_cast<const uint4*>(blk + n * MROWB + ((c ^ tsw(n)) << 4));
        *reinterpret_cast<uint4*>(ob + (size_t)n * a.D * 2 + c * 16) = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_mconv(const ConvArgs& a, hipStream_t s, const LaunchTiming* t) {
  if (a.N > ML || a.N < 1 || a.d % MCG != 0 || a.ng != a.d / MCG) return hipErrorInvalidValue;
  const int blocks = a.B * a.H * a.ng;
  if (a.N == ML) return launch_k(mconv_kernel<true>, dim3(blocks), dim3(MNTHR), 0, s, t, a);
  return launch_k(mconv_kernel<false>, dim3(blocks), dim3(MNTHR), 0, s, t, a);
}

}  // namespace cat
