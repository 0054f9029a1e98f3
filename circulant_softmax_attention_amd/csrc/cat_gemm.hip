// cat_gemm.hip -- the projections X . W on MFMA (gfx950).
//
// CAT projects the tokens with W_A (one score column per head) and W_V
// (CAT: Circular-Convolutional Attention for Sub-Quadratic Transformers,
// "Method details / Overall framework"); the ViT circulant attention projects
// them to Q, K and V (Vision Transformers are Circulant Attention Learners,
// "Circulant Attention: attention rebuilt with the FFT").  Both are one dense
// contraction Y = X W with X [M = B N][K = D] and W [D][ncols], run here as a
// single launch over up to three column segments (e.g. W_V and W_A), each
// written in the layout its consumer reads.
//
// Tiling: 128 x 128 output tile per 256-thread workgroup (4 waves, 2 x 2),
// each wave a 64 x 64 block of 16 x 16 MFMA tiles.  K is walked in tiles of
// two "K-chunks"; a K-chunk is what one lane feeds the MFMA from 16 bytes:
//   bf16: 8 values -> v_mfma_f32_16x16x32_bf16 (fp32 accumulate)
//   fp32: 4 values -> four v_mfma_f32_16x16x4_f32
// Every lane reads the same K positions for its A row and its B column, so
// the order in which the hardware walks K inside a chunk does not matter.
// X tiles are staged row-major in LDS; W tiles are transposed on the way in
// (K contiguous per output column) so both operands are 16-byte LDS reads.
// LDS is double buffered: the next tile is fetched into registers while the
// current one is multiplied.
#include "cat_common.hpp"
#include "cat_internal.hpp"

namespace cat {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

namespace {

constexpr int BM = 128, BN = 128, NTHR = 256;

template <int ET>
struct GemmCfg {
  static constexpr int ESZ = ET == ET_F32 ? 4 : 2;
  static constexpr int VE = 16 / ESZ;   // elements per 16-byte chunk
  static constexpr int KC = 4 * VE;     // K per chunk across the 4 lane groups
  static constexpr int BK = 2 * KC;     // K per LDS tile
  static constexpr int PITCH = BK + VE; // LDS row pitch (elements), +16 B pad
};

template <int ET>
__device__ __forceinline__ void store_out(const GemmSeg& s, const GemmArgs& a, int row, int col, float v) {
  size_t idx;
  if (s.layout == OUT_ROWMAJOR) {
    idx = (size_t)row * s.ncols + col;
  } else {
    const int b = row / a.Ntok, tok = row - b * a.Ntok;
    if (s.layout == OUT_HEADMAJOR) {
      idx = ((size_t)b * s.ncols + col) * a.Ntok + tok;
    } else {
      const int h = col / a.d, c = col - h * a.d;
      const int g = c / s.cg, j = c - g * s.cg;
      const int ng = a.d / s.cg;
      idx = (((size_t)(b * a.H + h) * ng + g) * a.Ntok + tok) * s.cg + j;
    }
  }
  if (s.out_f32 || ET == ET_F32) {
    reinterpret_cast<float*>(s.out)[idx] = v;
  } else {
    reinterpret_cast<uint16_t*>(s.out)[idx] = to_bf16(v);
  }
}

template <int ET>
__global__ __launch_bounds__(NTHR, 2) void gemm_xw_kernel(GemmArgs a) {
  using C = GemmCfg<ET>;
  constexpr int VE = C::VE, KC = C::KC, BK = C::BK, PITCH = C::PITCH;
  using elem_t = typename std::conditional<ET == ET_F32, float, uint16_t>::type;
  __shared__ __attribute__((aligned(16))) elem_t As[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) elem_t Bs[2][BN * PITCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int q = xcd_remap(blockIdx.x, gridDim.x);
  const int rt = q / a.ncoltiles;
  int ct = q - rt * a.ncoltiles;
  int si = 0;
  while (si + 1 < a.nseg && ct >= a.seg[si].ntiles) {
    ct -= a.seg[si].ntiles;
    ++si;
  }
  const GemmSeg& sg = a.seg[si];
  const int m0 = rt * BM, n0 = ct * BN;
  const int M = a.M, K = a.K, ncols = sg.ncols;
  const elem_t* X = reinterpret_cast<const elem_t*>(a.X);
  const elem_t* W = reinterpret_cast<const elem_t*>(sg.W);

  // A: 4 chunks of 16 B per thread, chunk c -> (row, 16-byte column); rows of
  // the tile are contiguous in X, so a wave reads whole 128-byte lines.
  constexpr int ACH = BK / VE;  // chunks per row
  // B: every thread reads 16 consecutive K rows of 4 bytes (2 bf16 columns or
  // 1 fp32 column), so a wave covers 256 contiguous bytes of one W row per
  // load; it then writes its columns K-contiguous into LDS.
  constexpr int CPT = 4 / C::ESZ;          // columns per thread
  constexpr int NCT = BN / CPT;            // threads along N
  constexpr int KR = BK / (NTHR / NCT);    // K rows per thread (16)
  static_assert(KR == 16, "B staging assumes 16 K rows per thread");
  const int bc = tid % NCT, bk = tid / NCT;
  const bool wvec = ET == ET_F32 || (ncols % 2) == 0;

  uint4 ra[4];
  uint32_t rb[KR];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + NTHR * i;
      const int row = c / ACH, kc = c - row * ACH;
      const int m = m0 + row, k = k0 + kc * VE;
      if (m < M && k < K) {
        ra[i] = *reinterpret_cast<const uint4*>(X + (size_t)m * K + k);
      } else {
        ra[i] = make_uint4(0, 0, 0, 0);
      }
    }
    const int n = n0 + bc * CPT;
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int k = k0 + KR * bk + r;
      if (k < K && n + CPT <= ncols && wvec) {
        rb[r] = *reinterpret_cast<const uint32_t*>(W + (size_t)k * ncols + n);
      } else {
        elem_t tmp[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) tmp[j] = (k < K && n + j < ncols) ? W[(size_t)k * ncols + n + j] : elem_t(0);
        rb[r] = *reinterpret_cast<uint32_t*>(tmp);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + NTHR * i;
      const int row = c / ACH, kc = c - row * ACH;
      *reinterpret_cast<uint4*>(&As[buf][row * PITCH + kc * VE]) = ra[i];
    }
    if constexpr (ET == ET_F32) {
      uint4* dst = reinterpret_cast<uint4*>(&Bs[buf][bc * PITCH + KR * bk]);
#pragma unroll
      for (int q4 = 0; q4 < KR / 4; ++q4)
        dst[q4] = make_uint4(rb[4 * q4], rb[4 * q4 + 1], rb[4 * q4 + 2], rb[4 * q4 + 3]);
    } else {
      // rb[r] holds (column n, column n+1) of row r; split into two K-runs
      uint32_t c0[KR / 2], c1[KR / 2];
#pragma unroll
      for (int r = 0; r < KR / 2; ++r) {
        const uint32_t a0 = rb[2 * r], a1 = rb[2 * r + 1];
        c0[r] = (a0 & 0xffffu) | (a1 << 16);
        c1[r] = (a0 >> 16) | (a1 & 0xffff0000u);
      }
      uint4* d0 = reinterpret_cast<uint4*>(&Bs[buf][(2 * bc) * PITCH + KR * bk]);
      uint4* d1 = reinterpret_cast<uint4*>(&Bs[buf][(2 * bc + 1) * PITCH + KR * bk]);
      d0[0] = make_uint4(c0[0], c0[1], c0[2], c0[3]);
      d0[1] = make_uint4(c0[4], c0[5], c0[6], c0[7]);
      d1[0] = make_uint4(c1[0], c1[1], c1[2], c1[3]);
      d1[1] = make_uint4(c1[4], c1[5], c1[6], c1[7]);
    }
  };

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int lrow = lane & 15, lgrp = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int kc = 0; kc < BK / KC; ++kc) {
      uint4 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const uint4*>(&As[buf][(wm * 64 + 16 * i + lrow) * PITCH + kc * KC + lgrp * VE]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const uint4*>(&Bs[buf][(wn * 64 + 16 * j + lrow) * PITCH + kc * KC + lgrp * VE]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (ET == ET_F32) {
            const float4 fa = *reinterpret_cast<const float4*>(&af[i]);
            const float4 fb = *reinterpret_cast<const float4*>(&bfr[j]);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.x, fb.x, acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.y, fb.y, acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.z, fb.z, acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.w, fb.w, acc[i][j], 0, 0, 0);
          } else {
            const bf16x8 va = *reinterpret_cast<const bf16x8*>(&af[i]);
            const bf16x8 vb = *reinterpret_cast<const bf16x8*>(&bfr[j]);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, vb, acc[i][j], 0, 0, 0);
          }
        }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // 16x16 MFMA result layout: lane holds column (lane & 15), rows 4 (lane >> 4) + v.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm * 64 + 16 * i + 4 * lgrp + v;
        const int col = n0 + wn * 64 + 16 * j + lrow;
        if (row < M && col < ncols) store_out<ET>(sg, a, row, col, acc[i][j][v]);
      }
}

}  // namespace

hipError_t launch_gemm(int et, GemmArgs a, hipStream_t stream) {
  a.ncoltiles = 0;
  for (int s = 0; s < a.nseg; ++s) {
    a.seg[s].ntiles = (a.seg[s].ncols + BN - 1) / BN;
    a.ncoltiles += a.seg[s].ntiles;
  }
  const int rowtiles = (a.M + BM - 1) / BM;
  const dim3 grid((unsigned)(rowtiles * a.ncoltiles)), block(NTHR);
  if (et == ET_F32) {
    hipLaunchKernelGGL(gemm_xw_kernel<ET_F32>, grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL(gemm_xw_kernel<ET_BF16>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace cat
