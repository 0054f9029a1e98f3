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
// current one is multiplied.  The finished tile goes through LDS once more so
// that every output store is a 16-byte vector in the consumer's layout.
#include "cat_common.hpp"
#include "cat_internal.hpp"

namespace cat {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

namespace {

constexpr int BM = 128, BN = 128, NTHR = 256;
constexpr int CP = BN + 4;  // fp32 pitch of the staged output tile

template <int ET>
struct GemmCfg {
  static constexpr int ESZ = ET == ET_F32 ? 4 : 2;
  static constexpr int VE = 16 / ESZ;   // elements per 16-byte chunk
  static constexpr int KC = 4 * VE;     // K per chunk across the 4 lane groups
  static constexpr int BK = 2 * KC;     // K per LDS tile
  static constexpr int PITCH = BK + VE; // LDS row pitch (elements), +16 B pad
  static constexpr int TILE_BYTES = 2 * 2 * 128 * PITCH * ESZ;  // A and B, two buffers
  static constexpr int SMEM = TILE_BYTES > BM * CP * 4 ? TILE_BYTES : BM * CP * 4;
};

// Element offset of output (row, col) of segment s.
__device__ __forceinline__ size_t out_index(const GemmSeg& s, const GemmArgs& a, int row, int col) {
  if (s.layout == OUT_ROWMAJOR) return (size_t)row * s.ncols + col;
  const uint32_t b = fastdiv((uint32_t)row, a.fd_ntok);
  const uint32_t tok = (uint32_t)row - b * (uint32_t)a.Ntok;
  if (s.layout == OUT_HEADMAJOR) return ((size_t)b * s.ncols + col) * a.Ntok + tok;
  const uint32_t h = fastdiv((uint32_t)col, a.fd_d);
  const uint32_t c = (uint32_t)col - h * (uint32_t)a.d;
  const uint32_t g = fastdiv(c, s.fd_cg);
  const uint32_t j = c - g * (uint32_t)s.cg;
  const uint32_t ng = (uint32_t)a.d / (uint32_t)s.cg;
  return (((size_t)(b * a.H + h) * ng + g) * a.Ntok + tok) * s.cg + j;
}

template <int ET>
__global__ __launch_bounds__(NTHR, 2) void gemm_xw_kernel(GemmArgs a) {
  using C = GemmCfg<ET>;
  constexpr int VE = C::VE, KC = C::KC, BK = C::BK, PITCH = C::PITCH;
  using elem_t = typename std::conditional<ET == ET_F32, float, uint16_t>::type;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  elem_t* As0 = reinterpret_cast<elem_t*>(smem);
  elem_t* Bs0 = As0 + 2 * 128 * PITCH;
  float* Cs = reinterpret_cast<float*>(smem);

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
  const GemmSeg sg = a.seg[si];
  const int m0 = rt * BM, n0 = ct * BN;
  const int M = a.M, K = a.K, ncols = sg.ncols;

  // A: 4 chunks of 16 B per thread: row = tid/8 + 32 i, column chunk tid % 8.
  constexpr int ACH = BK / VE;
  static_assert(ACH == 8, "A staging assumes 8 chunks per row");
  const int arow = tid / ACH, akc = tid % ACH;
  const elem_t* aptr[4];
  bool aok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + arow + 32 * i;
    aok[i] = m < M;
    aptr[i] = reinterpret_cast<const elem_t*>(a.X) + (size_t)(aok[i] ? m : 0) * K + akc * VE;
  }
  // B: every thread reads 16 consecutive K rows of 4 bytes (2 bf16 columns or
  // 1 fp32 column), so a wave covers 256 contiguous bytes of one W row per
  // load; it then writes its columns K-contiguous into LDS.
  constexpr int CPT = 4 / C::ESZ;
  constexpr int NCT = BN / CPT;
  constexpr int KR = BK / (NTHR / NCT);
  static_assert(KR == 16, "B staging assumes 16 K rows per thread");
  const int bc = tid % NCT, bk = tid / NCT;
  const int bn = n0 + bc * CPT;
  const elem_t* bptr = reinterpret_cast<const elem_t*>(sg.W) + (size_t)(KR * bk) * ncols + bn;

  uint4 ra[4];
  uint32_t rb[KR];
  // Interior tiles (the whole tile inside M x ncols, K a multiple of BK, W
  // rows 4-byte aligned) take unconditional vector loads; edge tiles take the
  // guarded path.  The choice is uniform across the workgroup, so the loads
  // of a tile are issued back to back with no waits between them.
  const bool full = (m0 + BM <= M) && (n0 + BN <= ncols) && (K % BK == 0) &&
                    (ET == ET_F32 || (ncols % 2) == 0);
  auto gload_full = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const uint4*>(aptr[i] + k0);
    const elem_t* bp = bptr + (size_t)k0 * ncols;
#pragma unroll
    for (int r = 0; r < KR; ++r) rb[r] = *reinterpret_cast<const uint32_t*>(bp + (size_t)r * ncols);
  };
  // Edge tiles: indices are clamped into range so every load is in bounds,
  // and out-of-range elements are zeroed by a select (no branch per load).
  auto gload_edge = [&](int k0) {
    const int kk = k0 + akc * VE < K ? k0 : K - VE - akc * VE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(aptr[i] + kk);
      ra[i] = (aok[i] & (k0 + akc * VE < K)) ? v : make_uint4(0, 0, 0, 0);
    }
    const elem_t* W = reinterpret_cast<const elem_t*>(sg.W);
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int k = k0 + KR * bk + r;
      const int kc = k < K ? k : K - 1;
      elem_t tmp[CPT];
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int n = bn + j < ncols ? bn + j : ncols - 1;
        const elem_t v = W[(size_t)kc * ncols + n];
        tmp[j] = ((k < K) & (bn + j < ncols)) ? v : elem_t(0);
      }
      rb[r] = *reinterpret_cast<uint32_t*>(tmp);
    }
  };
  auto gload = [&](int k0) {
    if (full) gload_full(k0);
    else gload_edge(k0);
  };
  auto lstore = [&](int buf) {
    elem_t* As = As0 + buf * 128 * PITCH;
    elem_t* Bs = Bs0 + buf * 128 * PITCH;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&As[(arow + 32 * i) * PITCH + akc * VE]) = ra[i];
    if constexpr (ET == ET_F32) {
      uint4* dst = reinterpret_cast<uint4*>(&Bs[bc * PITCH + KR * bk]);
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
      uint4* d0 = reinterpret_cast<uint4*>(&Bs[(2 * bc) * PITCH + KR * bk]);
      uint4* d1 = reinterpret_cast<uint4*>(&Bs[(2 * bc + 1) * PITCH + KR * bk]);
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
    const elem_t* As = As0 + buf * 128 * PITCH;
    const elem_t* Bs = Bs0 + buf * 128 * PITCH;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int kc = 0; kc < BK / KC; ++kc) {
      uint4 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const uint4*>(&As[(wm * 64 + 16 * i + lrow) * PITCH + kc * KC + lgrp * VE]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const uint4*>(&Bs[(wn * 64 + 16 * j + lrow) * PITCH + kc * KC + lgrp * VE]);
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

  // Stage the tile: 16x16 MFMA result layout is column (lane & 15),
  // rows 4 (lane >> 4) + v.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        Cs[(wm * 64 + 16 * i + 4 * lgrp + v) * CP + wn * 64 + 16 * j + lrow] = acc[i][j][v];
  __syncthreads();

  // One 16-byte output chunk of cr x cc elements per step; the chunk shape
  // keeps the chunk contiguous in the segment's layout.
  const bool f32out = sg.out_f32 || ET == ET_F32;
  const int VO = f32out ? 4 : 8;
  const int cr = sg.cr, cc = sg.cc;
  const int nrc = BM / cr, ncc = BN / cc;
  const bool rows_fast = sg.layout != OUT_ROWMAJOR;
  for (int qq = tid; qq < nrc * ncc; qq += NTHR) {
    const int rci = rows_fast ? qq % nrc : qq / ncc;
    const int cci = rows_fast ? qq / nrc : qq % ncc;
    const int lr = rci * cr, lc = cci * cc;
    const int row = m0 + lr, col = n0 + lc;
    if (row >= M || col >= ncols) continue;
    bool vec = row + cr <= M && col + cc <= ncols;
    size_t idx = out_index(sg, a, row, col);
    if (vec && cr > 1) {
      const uint32_t b = fastdiv((uint32_t)row, a.fd_ntok);
      vec = (uint32_t)(row + cr - 1) < (b + 1) * (uint32_t)a.Ntok;  // same sequence
    }
    vec = vec && (idx % VO) == 0;
    if (vec) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (e < VO) {
          const int er = e / cc, ec = e - er * cc;
          v[e] = Cs[(lr + er) * CP + lc + ec];
        }
      }
      if (f32out) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(sg.out) + idx) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(sg.out) + idx) =
            make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7]));
      }
    } else {
      for (int er = 0; er < cr; ++er)
        for (int ec = 0; ec < cc; ++ec) {
          const int r = row + er, c = col + ec;
          if (r >= M || c >= ncols) continue;
          const size_t o = out_index(sg, a, r, c);
          const float val = Cs[(lr + er) * CP + lc + ec];
          if (f32out) reinterpret_cast<float*>(sg.out)[o] = val;
          else reinterpret_cast<uint16_t*>(sg.out)[o] = to_bf16(val);
        }
    }
  }
}

// Score projection z[b][h][tok] = sum_k X[b tok][k] W_A[k][h] for the H score
// columns, on MFMA in 16-column blocks (CAT: Circular-Convolutional Attention
// for Sub-Quadratic Transformers, "Key designs: circulant attention matrix
// construction": Z = X W_A, one column per head).  A narrow product, so it is
// a kernel of its own: each wave owns 16 tokens and reads its A fragments
// straight from global memory; the 16 W_A columns of the block sit in LDS,
// transposed to K-contiguous rows, zero beyond H and beyond K.
constexpr int ZP_WAVES = 4;
template <int ET>
__global__ __launch_bounds__(ZP_WAVES * 64) void zproj_kernel(ZprojArgs a) {
  using C = GemmCfg<ET>;
  constexpr int VE = C::VE, KC = C::KC;
  using elem_t = typename std::conditional<ET == ET_F32, float, uint16_t>::type;
  extern __shared__ __attribute__((aligned(16))) char zsm[];
  elem_t* Bt = reinterpret_cast<elem_t*>(zsm);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, H = a.H, M = a.M;
  const int nsteps = (K + KC - 1) / KC;
  const int PB = nsteps * KC + VE;  // LDS pitch (elements) of one column
  const int c0 = blockIdx.y * 16;
  const elem_t* W = reinterpret_cast<const elem_t*>(a.W);
  // W_A[:, c0 : c0+16] -> Bt[c][k], sixteen loads in flight per thread
  const int total = 16 * PB;
  for (int base = 0; base < total; base += 16 * ZP_WAVES * 64) {
    elem_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int idx = base + u * ZP_WAVES * 64 + tid;
      const int c = idx / PB, k = idx - c * PB;
      const bool ok = (idx < total) & (k < K) & (c0 + c < H);
      const int kk = k < K ? k : K - 1, cc = c0 + c < H ? c0 + c : H - 1;
      const elem_t w = W[(size_t)kk * H + cc];
      v[u] = ok ? w : elem_t(0);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int idx = base + u * ZP_WAVES * 64 + tid;
      if (idx < total) Bt[idx] = v[u];
    }
  }
  __syncthreads();

  const int lrow = lane & 15, lgrp = lane >> 4;
  const int row = blockIdx.x * (ZP_WAVES * 16) + wave * 16 + lrow;
  const int rowc = row < M ? row : M - 1;
  const elem_t* xr = reinterpret_cast<const elem_t*>(a.X) + (size_t)rowc * K;
  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
  constexpr int ZB = 16;  // A fragments in flight per wave
  for (int s0 = 0; s0 < nsteps; s0 += ZB) {
    uint4 af[ZB];
#pragma unroll
    for (int u = 0; u < ZB; ++u) {
      const int k = (s0 + u) * KC + lgrp * VE;
      const int kk = k < K ? k : K - VE;
      const uint4 v = *reinterpret_cast<const uint4*>(xr + kk);
      af[u] = ((k < K) & (row < M)) ? v : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < ZB; ++u) {
      if (s0 + u < nsteps) {
        const uint4 bv = *reinterpret_cast<const uint4*>(&Bt[lrow * PB + (s0 + u) * KC + lgrp * VE]);
        if constexpr (ET == ET_F32) {
          const float4 fa = *reinterpret_cast<const float4*>(&af[u]);
          const float4 fb = *reinterpret_cast<const float4*>(&bv);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.x, fb.x, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.y, fb.y, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.z, fb.z, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.w, fb.w, acc, 0, 0, 0);
        } else {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(&af[u]),
                                                        *reinterpret_cast<const bf16x8*>(&bv), acc, 0, 0, 0);
        }
      }
    }
  }
  // result: column (lane & 15) = head c0 + lrow, rows 4 lgrp + v of the wave
  const int head = c0 + lrow;
  if (head < H) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = blockIdx.x * (ZP_WAVES * 16) + wave * 16 + 4 * lgrp + v;
      if (r < M) {
        const uint32_t b = fastdiv((uint32_t)r, a.fd_ntok);
        const uint32_t tok = (uint32_t)r - b * (uint32_t)a.Ntok;
        a.z[((size_t)b * H + head) * a.Ntok + tok] = acc[v];
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(int et, GemmArgs a, hipStream_t stream) {
  a.ncoltiles = 0;
  a.fd_ntok = make_fastdiv((uint32_t)a.Ntok);
  a.fd_d = make_fastdiv((uint32_t)a.d);
  for (int s = 0; s < a.nseg; ++s) {
    GemmSeg& g = a.seg[s];
    g.ntiles = (g.ncols + BN - 1) / BN;
    a.ncoltiles += g.ntiles;
    const int vo = (g.out_f32 || et == ET_F32) ? 4 : 8;
    if (g.layout == OUT_ROWMAJOR) {
      g.cr = 1;
      g.cc = vo;
    } else if (g.layout == OUT_HEADMAJOR) {
      g.cr = vo;
      g.cc = 1;
    } else if (g.cg >= vo) {
      g.cr = 1;
      g.cc = vo;
    } else {
      g.cr = vo / g.cg;
      g.cc = g.cg;
    }
    g.fd_cg = make_fastdiv((uint32_t)(g.cg > 0 ? g.cg : 1));
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

size_t zproj_lds_bytes(int et, int K) {
  const int esz = et == ET_F32 ? 4 : 2;
  const int kc = 4 * (16 / esz), ve = 16 / esz;
  const int pb = ((K + kc - 1) / kc) * kc + ve;
  return (size_t)16 * pb * esz;
}

hipError_t prepare_zproj(int et, int K) {
  const size_t bytes = zproj_lds_bytes(et, K);
  if (et == ET_F32)
    return hipFuncSetAttribute((const void*)zproj_kernel<ET_F32>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  return hipFuncSetAttribute((const void*)zproj_kernel<ET_BF16>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_zproj(int et, ZprojArgs a, hipStream_t stream) {
  a.fd_ntok = make_fastdiv((uint32_t)a.Ntok);
  const dim3 grid((unsigned)((a.M + ZP_WAVES * 16 - 1) / (ZP_WAVES * 16)), (unsigned)((a.H + 15) / 16));
  const size_t lds = zproj_lds_bytes(et, a.K);
  if (et == ET_F32) {
    hipLaunchKernelGGL(zproj_kernel<ET_F32>, grid, dim3(ZP_WAVES * 64), lds, stream, a);
  } else {
    hipLaunchKernelGGL(zproj_kernel<ET_BF16>, grid, dim3(ZP_WAVES * 64), lds, stream, a);
  }
  return hipGetLastError();
}

}  // namespace cat
