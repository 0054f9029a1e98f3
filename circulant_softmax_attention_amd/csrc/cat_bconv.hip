// cat_bconv.hip -- the 2D BCCB mixing on the matrix cores (gfx950, bf16
// storage, square grids of 32 or 96 tokens a side).
//
// The circulant-attention page evaluates O_h = BCCB(a*_h) V_h as a 2D
// circular convolution through 2D FFTs (Vision Transformers are Circulant
// Attention Learners, "Circulant Attention: attention rebuilt with the
// FFT").  On a G x G grid the 2D DFT is separable and has no twiddles: it is
// F X F with the dense G x G DFT matrix F[j][k] = w^(j k), w = e^(-2 pi i / G),
// so each 1D pass over the whole grid is one G x G x G complex matrix
// product.  Two real channels c, c' form one complex grid c + i c' (the
// filter is real, so one complex convolution gives both).  Per grid, with
// r, c the token row and column and kr, kc their frequencies:
//
//   pass 1 (over c):   D1[r][kc]  = sum_c X[r][c] F[c][kc]
//   pass 2 (over r):   D2[kr][kc] = sum_r F[kr][r] D1[r][kc]
//   spectrum product:  Z[kr][kc]  = D2[kr][kc] S[kr][kc]     (S = DFT2(a*) / N)
//   pass 3 (over kr):  D3[kc][r'] = sum_kr Z[kr][kc] conj F[kr][r']
//   pass 4 (over kc):  O[r'][c']  = sum_kc D3[kc][r'] conj F[kc][c']
//
// Every product runs as v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32
// accumulation), four real MFMAs per complex 16 x 16 x 32 block.  bf16 keeps
// fp32's range, so no block scaling is needed; each operand rounding costs
// 2^-9 relative, about 4e-3 relative L2 over the four passes (the bf16
// storage bar is 2e-2).  An MFMA result holds its row index in registers (4
// rows per lane group) and its column index across the 16 lanes of a group,
// which is how the next MFMA's operand holds its contracted and its kept
// index: passes 1 -> 2 -> 3 chain in registers, each contracting the previous
// result's row index, by using the data alternately as the A operand (kept
// index = rows) and as the B operand (kept index = columns).  K slot s of
// lane group g stands for index 4 g + (s mod 4) + 16 (s / 4) within a K step
// of 32, the order a result's rows come in; the constant operands use the
// same order.  Signs live on the data operands: the constant fragments are
// used as stored (real and imaginary parts only), each data operand carries
// the negated part its products need (-im for the forward transform, -re
// for the inverse), and the (-1)^k that separates DFT rows j and j + G/2
// becomes a sign flip of the data's odd K slots, applied in place once the
// lower-half tiles are done.
//
// Work split: a workgroup of eight waves takes four channel pairs of one
// head (8 channels); waves w and w + 4 carry pair w through passes 1-3 in
// the pair's LDS buffer.  Pass 1 streams the pair's block from memory once,
// row tile by row tile (the two waves take alternate row tiles), and writes
// D1 kc-major (rows kc, 16-column bands = kc tiles); passes 2-3 then take
// one band at a time (alternate bands per wave), reading its D1 rows and
// writing the band's D3 rows in their place.  Pass 4 contracts kc, so it
// waits for all four buffers and is split by output tiles over the eight
// waves: its D3 operand (kc in the K slots, one r' per lane) comes from
// transposing LDS reads of the kc-major buffer, and each lane produces one
// token for all four pairs, a 16-byte store of 8 channels per token into O
// [B][N][D].  Two waves per SIMD hide each other's LDS and memory waits;
// the constant fragments (real and imaginary parts) stay in registers.
//
// Layouts: V BLOCKED with 2-channel groups ([B][H][d/2][N][2], one pair's
// grid contiguous); S [BH][kr][kc] complex fp32 with kc contiguous; the DFT
// table [tile i][K step][re/im][lane][8 slots] bf16 for tiles i < G/32,
// made by the plan; O [B][N][D].
#include "cat_common.hpp"
#include "cat_internal.hpp"

namespace cat {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

namespace {

constexpr int BT = 512;  // eight waves, four channel pairs

template <int G>
struct BC {
  static constexpr int NT = G / 16;        // 16-wide tiles per side
  static constexpr int KS = G / 32;        // K steps of 32 per contraction
  static constexpr int NH = NT / 2;        // tiles in one half (rows j and j + G/2 differ by (-1)^k)
  static constexpr int PITCH = G + 8;      // bf16 per LDS row (208 bytes at G = 96)
  static constexpr int PLANE = G * PITCH;  // bf16 per plane
  static_assert(G % 32 == 0, "grid side");
};

// 8 values (one K-slot run) of one part as raw bits.
typedef uint4 raw8;
// A data operand: real and imaginary parts and the negated part its products
// take (-im in the forward transform, -re in the inverse).
struct CX {
  raw8 re, im, n;
};
struct KF {  // a constant fragment
  raw8 re, im;
};
struct CT {
  floatx4 re, im;
};

__device__ __forceinline__ floatx4 mm(const raw8& a, const raw8& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}
__device__ __forceinline__ raw8 xr8(const raw8& x, uint32_t m) { return make_uint4(x.x ^ m, x.y ^ m, x.z ^ m, x.w ^ m); }
constexpr uint32_t NEG = 0x80008000u;  // every slot negated
constexpr uint32_t ODD = 0x80000000u;  // odd slots (high halves) negated

// Forward data operand from its parts; the inverse one.
__device__ __forceinline__ CX fwd(const raw8& re, const raw8& im) { return CX{re, im, xr8(im, NEG)}; }
__device__ __forceinline__ CX inv(const raw8& re, const raw8& im) { return CX{re, im, xr8(re, NEG)}; }
// The odd-slot flip, in place: (-1)^k on the data stands for the upper-half
// DFT tile (rows j + G / 2) of the constant it meets.
__device__ __forceinline__ void flip(CX& d) {
  d.re = xr8(d.re, ODD);
  d.im = xr8(d.im, ODD);
  d.n = xr8(d.n, ODD);
}

// acc += data (A operand, rows kept) x constant (B):
//   forward (n = -di):  (dr + i di)(kr + i ki) = dr kr + (-di) ki + i (dr ki + di kr)
//   inverse (n = -dr):  (dr + i di)(kr - i ki) = dr kr + di ki + i (di kr + (-dr) ki)
__device__ __forceinline__ void mulA_f(const CX& d, const KF& k, CT& acc) {
  acc.re = mm(d.n, k.im, mm(d.re, k.re, acc.re));
  acc.im = mm(d.im, k.re, mm(d.re, k.im, acc.im));
}
__device__ __forceinline__ void mulA_i(const CX& d, const KF& k, CT& acc) {
  acc.re = mm(d.im, k.im, mm(d.re, k.re, acc.re));
  acc.im = mm(d.n, k.im, mm(d.im, k.re, acc.im));
}
// acc += constant (A) x data (B operand, columns kept), same forms.
__device__ __forceinline__ void mulB_f(const KF& k, const CX& d, CT& acc) {
  acc.re = mm(k.im, d.n, mm(k.re, d.re, acc.re));
  acc.im = mm(k.im, d.re, mm(k.re, d.im, acc.im));
}
__device__ __forceinline__ void mulB_i(const KF& k, const CX& d, CT& acc) {
  acc.re = mm(k.im, d.im, mm(k.re, d.re, acc.re));
  acc.im = mm(k.im, d.n, mm(k.re, d.im, acc.im));
}
// Parts of a K operand whose slot v + 4 y takes value v of tile y, rounded to bf16.
__device__ __forceinline__ raw8 stack_re(const CT& t0, const CT& t1) {
  return make_uint4(pack_bf16x2(t0.re[0], t0.re[1]), pack_bf16x2(t0.re[2], t0.re[3]), pack_bf16x2(t1.re[0], t1.re[1]),
                    pack_bf16x2(t1.re[2], t1.re[3]));
}
__device__ __forceinline__ raw8 stack_im(const CT& t0, const CT& t1) {
  return make_uint4(pack_bf16x2(t0.im[0], t0.im[1]), pack_bf16x2(t0.im[2], t0.im[3]), pack_bf16x2(t1.im[0], t1.im[1]),
                    pack_bf16x2(t1.im[2], t1.im[3]));
}
// Two pair words (re | im << 16 each) -> the low halves and the high halves.
__device__ __forceinline__ uint32_t lo2(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t hi2(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }
__device__ __forceinline__ CT zero_ct() {
  CT c;
  c.re = floatx4{0.f, 0.f, 0.f, 0.f};
  c.im = floatx4{0.f, 0.f, 0.f, 0.f};
  return c;
}

// Transposing LDS read (gfx950): lane L of each 16-lane group supplies the
// address of row k0 + L / 4, columns x0 + 4 (L % 4) .. + 3 of a row-major
// bf16 tile; it receives rows k0 .. k0 + 3 of column x0 + L.
__device__ __forceinline__ uint2 ds_tr(const uint16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(const __attribute__((address_space(3))) char*)p);
  return __builtin_bit_cast(uint2, r);
}

// Work units: a.nfull quads (four pairs, 16-byte stores of 8 channels per
// token), then a.nhalf half-quads (two pairs, 8-byte stores) that continue
// the order (b, h, pair) after the quads; the workgroups stride over each
// list.  A unit of NPW pairs has 8 / NPW waves per pair.
template <int G>
__global__ __launch_bounds__(BT) void bconv_kernel(BconvArgs a) {
  using P = BC<G>;
  constexpr int NT = P::NT, KS = P::KS, NH = P::NH, PITCH = P::PITCH, PLANE = P::PLANE;
  constexpr int N = G * G;
  // per pair, kc-major planes (re, im) [kc][x], bf16: D1 (x = r) after pass 1;
  // pass 3 overwrites band kt with D3 (x = r') once pass 2 has read it
  __shared__ __attribute__((aligned(16))) uint16_t es[4][2 * PLANE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lo = lane & 15, grp = lane >> 4;

  // DFT fragments kf[i][t] for i < NH: lane (lo, grp), slot s ->
  // F[lo + 16 i][32 t + 4 grp + s % 4 + 16 (s / 4)]; tile i + NH is tile i
  // times (-1)^k, k having the parity of s.
  KF kf[NH][KS];
#pragma unroll
  for (int i = 0; i < NH; ++i)
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      const uint4* src = reinterpret_cast<const uint4*>(a.table) + ((size_t)(i * KS + t) * 2) * 64 + lane;
      kf[i][t] = KF{src[0], src[64]};
    }

  const int uq0 = xcd_remap(blockIdx.x, gridDim.x);
  auto run_units = [&](auto npw, int u0, int nu) {
  constexpr int NPW = decltype(npw)::value;
  constexpr int WPP = 8 / NPW;                    // waves per pair
  const int pw = wave % NPW, half = wave / NPW;  // the wave's pair, and which of its waves
  const int upb = a.npair / NPW;                 // units per (b, h)
  for (int uq = uq0; uq < nu; uq += gridDim.x) {
    const int q = u0 + uq;
    const int bh = q / upb, pq = q - bh * upb;  // unit pq: pairs NPW pq ..
    const int b = bh / a.H, h = bh - b * a.H;
    const float2* spec = a.spec + (size_t)bh * N;
    uint16_t* e = es[pw];

    // ---- pass 1 (pair NPW pq + pw, row tiles half, half + WPP, ...): the
    // pair's words streamed from memory once (two row tiles in flight), D1
    // of all kc tiles written to LDS
    {
      const uint32_t* vp = reinterpret_cast<const uint32_t*>(a.V) + ((size_t)bh * a.npair + NPW * pq + pw) * N;
      uint4 w[2][KS][2];
      auto fetch = [&](int slot, int ri) {
#pragma unroll
        for (int t = 0; t < KS; ++t) {
          const uint32_t* row = vp + (size_t)(16 * ri + lo) * G + 32 * t + 4 * grp;
          w[slot][t][0] = *reinterpret_cast<const uint4*>(row);       // c = 32 t + 4 grp + 0..3
          w[slot][t][1] = *reinterpret_cast<const uint4*>(row + 16);  // c + 16
        }
      };
      constexpr int NJ = (NT + WPP - 1) / WPP;
      if (half < NT) fetch(0, half);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int ri = half + WPP * j;
        if (ri >= NT) break;  // uniform across the wave
        CX x[KS];
#pragma unroll
        for (int t = 0; t < KS; ++t) {
          const uint4 w0 = w[j & 1][t][0], w1 = w[j & 1][t][1];
          x[t] = fwd(make_uint4(lo2(w0.x, w0.y), lo2(w0.z, w0.w), lo2(w1.x, w1.y), lo2(w1.z, w1.w)),
                     make_uint4(hi2(w0.x, w0.y), hi2(w0.z, w0.w), hi2(w1.x, w1.y), hi2(w1.z, w1.w)));
        }
        if (j + 1 < NJ && ri + WPP < NT) fetch((j + 1) & 1, ri + WPP);
#pragma unroll
        for (int kt = 0; kt < NT; ++kt) {
          if (kt == NH) {
#pragma unroll
            for (int t = 0; t < KS; ++t) flip(x[t]);
          }
          CT d1 = zero_ct();
#pragma unroll
          for (int t = 0; t < KS; ++t) mulA_f(x[t], kf[kt < NH ? kt : kt - NH][t], d1);
          // rows r = 16 ri + 4 grp + v, col kc = 16 kt + lo -> es[kc][r .. r + 3]
          const int o = (16 * kt + lo) * PITCH + 16 * ri + 4 * grp;
          *reinterpret_cast<uint2*>(e + o) = make_uint2(pack_bf16x2(d1.re[0], d1.re[1]), pack_bf16x2(d1.re[2], d1.re[3]));
          *reinterpret_cast<uint2*>(e + PLANE + o) =
              make_uint2(pack_bf16x2(d1.im[0], d1.im[1]), pack_bf16x2(d1.im[2], d1.im[3]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();  // both waves' row tiles of each pair

    // ---- passes 2-3, one kc band at a time (band kt: rows 16 kt .. 16 kt +
    // 15), every WPP-th band per wave
#pragma unroll 1
    for (int kt = half; kt < NT; kt += WPP) {
      // pass 2 operand: D1[r slots][kc lanes] from the band's rows
      CX y[KS];
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        const int o = (16 * kt + lo) * PITCH + 32 * t + 4 * grp;  // r = 32 t + 4 grp + 0..3 and + 16
        const uint2 r0 = *reinterpret_cast<const uint2*>(e + o), r1 = *reinterpret_cast<const uint2*>(e + o + 16);
        const uint2 i0 = *reinterpret_cast<const uint2*>(e + PLANE + o),
                    i1 = *reinterpret_cast<const uint2*>(e + PLANE + o + 16);
        y[t] = fwd(make_uint4(r0.x, r0.y, r1.x, r1.y), make_uint4(i0.x, i0.y, i1.x, i1.y));
      }
      // pass 2 (rows kr = 16 ki + 4 grp + v, cols kc), each kr tile times the
      // spectrum S[kr][kc] (kc = 16 kt + lo), two tiles stacked into pass 3's
      // operand
      const float2* sk = spec + 16 * kt + lo + (size_t)(4 * grp) * G;
      raw8 zre[KS], zim[KS];
      CT dprev;
#pragma unroll
      for (int ki = 0; ki < NT; ++ki) {
        float2 sv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) sv[v] = sk[(size_t)(16 * ki + v) * G];
        if (ki == NH) {
#pragma unroll
          for (int t = 0; t < KS; ++t) flip(y[t]);
        }
        CT d2 = zero_ct();
#pragma unroll
        for (int t = 0; t < KS; ++t) mulB_f(kf[ki < NH ? ki : ki - NH][t], y[t], d2);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float xr = d2.re[v], xi = d2.im[v];
          d2.re[v] = fmaf(xr, sv[v].x, -xi * sv[v].y);
          d2.im[v] = fmaf(xr, sv[v].y, xi * sv[v].x);
        }
        if (ki & 1) {
          zre[ki / 2] = stack_re(dprev, d2);
          zim[ki / 2] = stack_im(dprev, d2);
        } else {
          dprev = d2;
        }
      }
      // pass 3 (data as B): D3[i] rows r' = 16 i + 4 grp + v, cols kc = 16 kt + lo
      // -> es[kc][r' .. r' + 3] (the band's rows, already read above)
      CX z[KS];
#pragma unroll
      for (int t = 0; t < KS; ++t) z[t] = inv(zre[t], zim[t]);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if (i == NH) {
#pragma unroll
          for (int t = 0; t < KS; ++t) flip(z[t]);
        }
        CT d3 = zero_ct();
#pragma unroll
        for (int t = 0; t < KS; ++t) mulB_i(kf[i < NH ? i : i - NH][t], z[t], d3);
        const int o = (16 * kt + lo) * PITCH + 16 * i + 4 * grp;
        *reinterpret_cast<uint2*>(e + o) = make_uint2(pack_bf16x2(d3.re[0], d3.re[1]), pack_bf16x2(d3.re[2], d3.re[3]));
        *reinterpret_cast<uint2*>(e + PLANE + o) =
            make_uint2(pack_bf16x2(d3.im[0], d3.im[1]), pack_bf16x2(d3.im[2], d3.im[3]));
      }
    }
    __syncthreads();

    // ---- pass 4: output tiles (rt, ct) of the unit's pairs; wave w takes
    // the tiles w, w + 8, ...  D4 rows r' = 16 rt + 4 grp + v, cols c' = 16 ct + lo.
    // Operand: D3[r' lanes][kc slots] by transposing reads of the kc-major planes.
    {
      uint16_t* ob = reinterpret_cast<uint16_t*>(a.O) + (size_t)b * N * a.D + (size_t)h * a.d + 2 * NPW * pq;
#pragma unroll 1
      for (int u = wave; u < NT * NT; u += 8) {
        const int rt = u / NT, ct = u - rt * NT;
        // column tile ct's constant: one of the fragments in registers,
        // chosen by a wave-uniform branch (a runtime index would send the
        // fragments to scratch), (-1)^k of the upper half applied
        const int c0 = ct < NH ? ct : ct - NH;
        const uint32_t fl = ct < NH ? 0u : ODD;
        auto tile = [&](const KF* kc) {
          uint32_t wv[4][NPW];  // [v][pair]
#pragma unroll
          for (int pp = 0; pp < NPW; ++pp) {
            CT d4 = zero_ct();
#pragma unroll
            for (int t = 0; t < KS; ++t) {
              // slots 0..3: kc = 32 t + 4 grp + 0..3; slots 4..7: kc + 16;
              // lane lo addresses row kc0 + lo / 4, columns 16 rt + 4 (lo % 4) ..
              const int o = (32 * t + 4 * grp + (lo >> 2)) * PITCH + 16 * rt + 4 * (lo & 3);
              const uint2 r0 = ds_tr(es[pp] + o), r1 = ds_tr(es[pp] + o + 16 * PITCH);
              const uint2 i0 = ds_tr(es[pp] + PLANE + o), i1 = ds_tr(es[pp] + PLANE + o + 16 * PITCH);
              mulA_i(inv(make_uint4(r0.x, r0.y, r1.x, r1.y), make_uint4(i0.x, i0.y, i1.x, i1.y)), kc[t], d4);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) wv[v][pp] = pack_bf16x2(d4.re[v], d4.im[v]);
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int n = (16 * rt + 4 * grp + v) * G + 16 * ct + lo;
            if constexpr (NPW == 4)
              *reinterpret_cast<uint4*>(ob + (size_t)n * a.D) = make_uint4(wv[v][0], wv[v][1], wv[v][2], wv[v][3]);
            else
              *reinterpret_cast<uint2*>(ob + (size_t)n * a.D) = make_uint2(wv[v][0], wv[v][1]);
          }
        };
        sfor<0, NH>([&](auto C) {
          if (c0 == decltype(C)::value) {
            KF kc[KS];
#pragma unroll
            for (int t = 0; t < KS; ++t) kc[t] = KF{xr8(kf[decltype(C)::value][t].re, fl), xr8(kf[decltype(C)::value][t].im, fl)};
            tile(kc);
          }
        });
      }
    }
    __syncthreads();  // es is rewritten by the next unit
  }
  };
  run_units(std::integral_constant<int, 4>{}, 0, a.nfull);
  run_units(std::integral_constant<int, 2>{}, 2 * a.nfull, a.nhalf);
}

}  // namespace

bool bconv_supported(int G) { return G == 32 || G == 96; }

size_t bconv_table_halfs(int G) { return (size_t)(G / 32) * (G / 32) * 2 * 64 * 8; }

hipError_t launch_bconv(const BconvArgs& a0, int G, hipStream_t s, const LaunchTiming* t) {
  if (!bconv_supported(G) || a0.d % 8 != 0 || a0.npair != a0.d / 2 || a0.BH < 1 || a0.table == nullptr ||
      a0.D % 8 != 0)
    return hipErrorInvalidValue;
  const long quads = (long)a0.BH * (a0.npair / 4);
  if (2 * quads > 0x7fffffffL) return hipErrorInvalidValue;
  // One workgroup per compute unit (four pairs' planes fill its LDS), each
  // looping over quads.  When the last round of quads would fill at most
  // half the compute units, those quads go as half-quads (two pairs each)
  // over all of them instead, so no compute unit idles through a whole
  // round.
  const long ncu = a0.num_cu > 0 ? a0.num_cu : 256;
  const long rem = quads % ncu;
  BconvArgs a = a0;
  a.nfull = (int)((rem > 0 && 2 * rem <= ncu) ? quads - rem : quads);
  a.nhalf = (int)(2 * (quads - a.nfull));
  long nb = a.nfull > a.nhalf ? a.nfull : a.nhalf;
  if (nb > ncu) nb = ncu;
  return launch_k(G == 96 ? bconv_kernel<96> : bconv_kernel<32>, dim3((unsigned)nb), dim3(BT), 0, s, t, a);
}

}  // namespace cat
