// cat_gemm.hip -- the projections X . W on MFMA (gfx950).
//
// CAT projects the tokens with W_A (one score column per head) and W_V
// (CAT: Circular-Convolutional Attention for Sub-Quadratic Transformers,
// "Method details / Overall framework"); the ViT circulant attention projects
// them to Q, K and V (Vision Transformers are Circulant Attention Learners,
// "Circulant Attention: attention rebuilt with the FFT").  Both are one dense
// contraction Y = X W with X [M = B N][K = D].  The GEMM reads W output-major,
// Wt [ncols][K] (each output channel's K weights contiguous); a small
// transpose kernel turns the input-major weights of the ABI into that layout
// once per call.  One launch covers up to three column segments, each
// written in the layout its consumer reads.
//
// Tiling: 128 x 128 output tile per 256-thread workgroup (4 waves, 2 x 2),
// each wave a 64 x 64 block of 16 x 16 MFMA tiles.  K is walked in tiles of
// 128 bytes per row (64 bf16 or 32 fp32 values), i.e. eight 16-byte chunks;
// a chunk is what one lane feeds the MFMA:
//   bf16: 8 values -> v_mfma_f32_16x16x32_bf16 (fp32 accumulate)
//   fp32: 4 values -> four v_mfma_f32_16x16x4_f32
// Every lane reads the same K positions for its A row and its B column, so
// the order in which the hardware walks K inside a chunk does not matter.
//
// Staging: both operand tiles are row-major [row][K] (X rows, Wt rows), so
// every chunk is one 16-byte load straight from global memory into LDS
// (LDS-DMA, no register round trip).  Rows are unpadded and the 16-byte
// position of chunk c in row r is c ^ (r % 8), which spreads the 16 rows of
// one fragment read over distinct banks.  Two LDS stages: the DMA of tile
// k + 1 is in flight while tile k is multiplied.  Rows beyond M or ncols are
// clamped to the last valid row (their results are never stored); a K tail
// that does not fill a tile goes through registers with the missing chunks
// zeroed.
//
// Score projection (1D): the workgroups of the first column tile also
// multiply their staged X rows by W_A^T (up to 32 heads, staged like a third
// operand of 32 rows), so z = X W_A costs no extra pass over X.  Each wave
// takes 32 of its 64 rows for this.
#include "cat_common.hpp"
#include "cat_internal.hpp"

namespace cat {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

namespace {

constexpr int BM = 128, NTHR = 256;
constexpr int ZR = 32;     // score-projection rows (heads) per stage
constexpr int ROWB = 128;  // bytes of one row of a K tile

template <int ET>
struct GemmCfg {
  static constexpr int ESZ = ET == ET_F32 ? 4 : 2;
  static constexpr int VE = 16 / ESZ;  // elements per 16-byte chunk
  static constexpr int BK = 8 * VE;    // K per tile (8 chunks, 128 bytes per row)
};

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One 16-byte LDS-DMA load per lane: lane l's 16 bytes at g land at LDS byte
// address lds + 16 l (lds must be uniform across the wave).  Written as
// inline asm so that the compiler adds no waits of its own before later LDS
// reads; completion is awaited explicitly with wait_vmem_all.
// M0 is reserved by the compiler, which only sets it right before the few
// instructions that read it, so declaring it clobbered here is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// acc += A^T B over one 16-byte chunk (A, B: 16 rows x chunk each; the
// result's column index follows B's rows).
template <int ET>
__device__ __forceinline__ floatx4 mfma_chunk(const uint4& ra, const uint4& rb, floatx4 acc) {
  if constexpr (ET == ET_F32) {
    const float4 fa = *reinterpret_cast<const float4*>(&ra);
    const float4 fb = *reinterpret_cast<const float4*>(&rb);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.x, fb.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.y, fb.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.z, fb.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.w, fb.w, acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(&ra),
                                                  *reinterpret_cast<const bf16x8*>(&rb), acc, 0, 0, 0);
  }
  return acc;
}

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

template <int ET, int BN>
__global__ __launch_bounds__(NTHR, 2) void gemm_xw_kernel(GemmArgs a) {
  using C = GemmCfg<ET>;
  constexpr int VE = C::VE, BK = C::BK;
  constexpr int STAGE = (BM + BN + ZR) * ROWB;  // one LDS stage: A rows, B rows, W_A^T rows
  constexpr int SMEM = 2 * STAGE;
  constexpr int BCH = BN * 8 / NTHR;            // B chunks per thread
  constexpr int TN = BN / 32;                   // 16-column MFMA blocks per wave
  static_assert(BCH * NTHR == BN * 8 && TN * 32 == BN, "tile width");
  using elem_t = typename std::conditional<ET == ET_F32, float, uint16_t>::type;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // Chunk slot s = tid + 256 i of an operand tile is row s / 8, 16-byte
  // position s % 8, and holds K-chunk (s % 8) ^ (row % 8) -- the same chunk
  // for every i, since row % 8 = (tid / 8) % 8.
  const int kch = ((tid & 7) ^ ((tid >> 3) & 7)) * VE;
  const elem_t* asrc[4];
  const elem_t* bsrc[BCH];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const int am = m0 + r < M ? m0 + r : M - 1;
    asrc[i] = reinterpret_cast<const elem_t*>(a.X) + (size_t)am * K + kch;
  }
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const int bn = n0 + r < ncols ? n0 + r : ncols - 1;
    bsrc[i] = reinterpret_cast<const elem_t*>(sg.W) + (size_t)bn * K + kch;
  }
  // score projection: W_A^T row tid / 8 (clamped; rows >= nz are never stored)
  const bool zwg = a.nz > 0 && si == 0 && ct == 0;
  const int nzb = (a.nz + 15) >> 4;
  const elem_t* zsrc = reinterpret_cast<const elem_t*>(a.Wz);
  if (zwg) {
    const int zr = (tid >> 3) < a.nz ? (tid >> 3) : a.nz - 1;
    zsrc += (size_t)zr * K + kch;
  }
  const uint32_t lds0 = lds_addr(smem) + (uint32_t)wave * 64 * 16;

  // Stage tile kt into LDS stage st.
  auto issue = [&](int kt, int st) {
    const int k0 = kt * BK;
    if (k0 + BK <= K) {
      const uint32_t base = lds0 + (uint32_t)(st * STAGE);
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_dma16(asrc[i] + k0, base + i * NTHR * 16);
#pragma unroll
      for (int i = 0; i < BCH; ++i) lds_dma16(bsrc[i] + k0, base + BM * ROWB + i * NTHR * 16);
      if (zwg) lds_dma16(zsrc + k0, base + (BM + BN) * ROWB);
    } else {
      // K tail: chunks at or beyond K are zero in both operands
      const bool ok = k0 + kch < K;
      const int kk = ok ? k0 : -kch;  // row start when the chunk is out of range
      uint4 va[4], vb[BCH];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(asrc[i] + kk);
        va[i] = ok ? v : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(bsrc[i] + kk);
        vb[i] = ok ? v : make_uint4(0, 0, 0, 0);
      }
      uint4* dst = reinterpret_cast<uint4*>(smem + st * STAGE) + tid;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i * NTHR] = va[i];
#pragma unroll
      for (int i = 0; i < BCH; ++i) dst[BM * 8 + i * NTHR] = vb[i];
      if (zwg) {
        const uint4 v = *reinterpret_cast<const uint4*>(zsrc + kk);
        dst[(BM + BN) * 8] = ok ? v : make_uint4(0, 0, 0, 0);
      }
    }
  };

  floatx4 acc[4][TN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  // zacc[ii][zb]: tokens of row block 2 wn + ii, heads 16 zb ..
  floatx4 zacc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) zacc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int lrow = lane & 15, lgrp = lane >> 4;
  const int sw = lrow & 7;  // row % 8 of every fragment row this lane reads
  // All fragments of both K-chunks are read first, so that the LDS latency of
  // the second chunk hides under the MFMAs of the first.
  auto compute = [&](int st) {
    const char* sa = smem + st * STAGE + (wm * 64 + lrow) * ROWB;
    const char* sb = smem + st * STAGE + BM * ROWB + (wn * (BN / 2) + lrow) * ROWB;
    uint4 af[2][4], bfr[2][TN];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int pos = ((kc * 4 + lgrp) ^ sw) * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) af[kc][i] = *reinterpret_cast<const uint4*>(sa + 16 * i * ROWB + pos);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[kc][j] = *reinterpret_cast<const uint4*>(sb + 16 * j * ROWB + pos);
    }
    // W fragment as the MFMA's A operand, X fragment as B: the 16 x 16 result
    // is Y^T, so each lane ends with 4 consecutive channels of one token (see
    // the stores below)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_chunk<ET>(bfr[kc][j], af[kc][i], acc[i][j]);
    if (zwg) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int pos = ((kc * 4 + lgrp) ^ sw) * 16;
        const char* sz = smem + st * STAGE + (BM + BN + lrow) * ROWB + pos;
#pragma unroll
        for (int zb = 0; zb < 2; ++zb) {
          if (zb < nzb) {
            const uint4 zf = *reinterpret_cast<const uint4*>(sz + 16 * zb * ROWB);
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
              const uint4 xa = wn ? af[kc][2 + ii] : af[kc][ii];  // no dynamic register indexing
              zacc[ii][zb] = mfma_chunk<ET>(zf, xa, zacc[ii][zb]);
            }
          }
        }
      }
    }
  };

  // Tile kt lives in stage kt % 2.  At the top of step kt every wave has its
  // own DMA of tile kt complete and, after the barrier, all of them have
  // finished multiplying tile kt - 1, whose stage then receives tile kt + 1.
  const int nk = (K + BK - 1) / BK;
  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmem_all();
    __syncthreads();
    if (kt + 1 < nk) issue(kt + 1, (kt + 1) & 1);
    compute(kt & 1);
  }
  // Result layout (16 x 16 MFMA, A = W rows, B = X rows): lane (lrow, lgrp)
  // holds Y[token][channel] for token = tile row base + lrow and the four
  // channels 4 lgrp + v, v = 0..3, of each 16-channel block.  Written
  // straight from registers: 8 (bf16) or 16 (fp32) bytes per lane, and the 16
  // lanes of a channel block cover 16 consecutive tokens.
  if (zwg) {
    // z [B][nz][Ntok] fp32: lane holds token lrow of its row block and heads
    // 16 zb + 4 lgrp + v; the 16 lanes of a head cover 16 consecutive tokens
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int token = m0 + wm * 64 + 16 * (2 * wn + ii) + lrow;
      if (token < M) {
        const uint32_t b = fastdiv((uint32_t)token, a.fd_ntok);
        const uint32_t tok = (uint32_t)token - b * (uint32_t)a.Ntok;
#pragma unroll
        for (int zb = 0; zb < 2; ++zb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int head = 16 * zb + 4 * lgrp + v;
            if (head < a.nz) a.z[((size_t)b * a.nz + head) * a.Ntok + tok] = zacc[ii][zb][v];
          }
      }
    }
  }
  const bool f32out = ET == ET_F32 || sg.out_f32;
  const bool quad = (sg.layout == OUT_ROWMAJOR && (ncols & 3) == 0) ||
                    (sg.layout == OUT_BLOCKED && (a.d & 3) == 0 && (sg.cg & 3) == 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int token = m0 + wm * 64 + 16 * i + lrow;
    if (token >= M) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int ch0 = n0 + wn * (BN / 2) + 16 * j + 4 * lgrp;
      if (ch0 >= ncols) continue;
      const floatx4 v = acc[i][j];
      if (quad && ch0 + 4 <= ncols) {
        const size_t o = out_index(sg, a, token, ch0);
        if (f32out) *reinterpret_cast<float4*>(reinterpret_cast<float*>(sg.out) + o) = make_float4(v[0], v[1], v[2], v[3]);
        else *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(sg.out) + o) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      } else if (sg.layout == OUT_BLOCKED && sg.cg == 2 && ch0 + 4 <= ncols) {
        // channel pairs (d is even, so a pair never straddles two heads)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const size_t o = out_index(sg, a, token, ch0 + 2 * p);
          if (f32out) *reinterpret_cast<float2*>(reinterpret_cast<float*>(sg.out) + o) = make_float2(v[2 * p], v[2 * p + 1]);
          else reinterpret_cast<uint32_t*>(sg.out)[o / 2] = pack_bf16x2(v[2 * p], v[2 * p + 1]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (ch0 + e >= ncols) break;
          const size_t o = out_index(sg, a, token, ch0 + e);
          if (f32out) reinterpret_cast<float*>(sg.out)[o] = v[e];
          else reinterpret_cast<uint16_t*>(sg.out)[o] = to_bf16(v[e]);
        }
      }
    }
  }
}

// Weight transpose W [rows][cols] -> W^T [cols][rows] through a 64 x 64 LDS
// tile, so that the GEMM can stage every operand row with 16-byte LDS-DMA.
// The weights are given input-major, X W as the pages write the projections;
// this pass turns them output-major once per call.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(TransposeArgs a) {
  constexpr int VE = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int P = sizeof(T) == 2 ? 66 : 65;  // LDS pitch (elements): column reads spread over banks
  __shared__ __attribute__((aligned(16))) T tile[64][P];
  const int tid = threadIdx.x;
  int b = blockIdx.x, m = 0;
  while (m + 1 < a.n && b >= a.tile0[m + 1]) ++m;
  b -= a.tile0[m];
  const int R = a.rows[m], Cc = a.cols[m];
  const int tcols = (Cc + 63) / 64;
  const int tr = b / tcols, tc = b - tr * tcols;
  const int r0 = tr * 64, c0 = tc * 64;
  const T* src = reinterpret_cast<const T*>(a.src[m]);
  T* dst = reinterpret_cast<T*>(a.dst[m]);
  // interior tiles move 16-byte chunks; edge tiles move single elements
  const bool full = (r0 + 64 <= R) & (c0 + 64 <= Cc) & (Cc % VE == 0) & (R % VE == 0);
  if (full) {
    constexpr int CPR = 64 / VE;        // chunks per 64-element row
    constexpr int NCH = 64 * CPR / 256;  // chunks per thread
    uint4 v[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = tid + 256 * i, r = q / CPR, ch = q % CPR;
      v[i] = *reinterpret_cast<const uint4*>(src + (size_t)(r0 + r) * Cc + c0 + ch * VE);
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = tid + 256 * i, r = q / CPR, ch = q % CPR;
      const T* e = reinterpret_cast<const T*>(&v[i]);
#pragma unroll
      for (int k = 0; k < VE; ++k) tile[r][ch * VE + k] = e[k];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = tid + 256 * i, c = q / CPR, ch = q % CPR;
      T e[VE];
#pragma unroll
      for (int k = 0; k < VE; ++k) e[k] = tile[ch * VE + k][c];
      *reinterpret_cast<uint4*>(dst + (size_t)(c0 + c) * R + r0 + ch * VE) = *reinterpret_cast<const uint4*>(e);
    }
    return;
  }
  const int lo = tid & 63, hi = tid >> 6;
  T v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + hi + 4 * i, c = c0 + lo;
    const bool ok = (r < R) & (c < Cc);
    const T x = src[(size_t)(r < R ? r : R - 1) * Cc + (c < Cc ? c : Cc - 1)];
    v[i] = ok ? x : T(0);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) tile[hi + 4 * i][lo] = v[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = c0 + hi + 4 * i, r = r0 + lo;
    if ((c < Cc) & (r < R)) dst[(size_t)c * R + r] = tile[lo][hi + 4 * i];
  }
}

// Output tile width: 128 or 96 columns.  Two workgroups fit a compute unit,
// so the grid runs in rounds of 2 x CUs workgroups; the width whose grid fills
// its last round best is taken (128 on a tie).
int choose_tile_n(const GemmArgs& a) {
  const int cus = a.num_cu > 0 ? a.num_cu : 256;
  const int rowtiles = (a.M + BM - 1) / BM;
  const long slots = 2L * cus;
  int best = 128;
  double best_fill = -1.0;
  for (int bn : {128, 96}) {
    long tiles = 0;
    for (int s = 0; s < a.nseg; ++s) tiles += (long)rowtiles * ((a.seg[s].ncols + bn - 1) / bn);
    const double fill = (double)tiles / (double)(((tiles + slots - 1) / slots) * slots);
    if (fill > best_fill + 1e-9) {
      best_fill = fill;
      best = bn;
    }
  }
  return best;
}

template <int BN>
hipError_t launch_gemm_bn(int et, GemmArgs& a, hipStream_t stream, const LaunchTiming* t) {
  a.ncoltiles = 0;
  for (int s = 0; s < a.nseg; ++s) {
    a.seg[s].ntiles = (a.seg[s].ncols + BN - 1) / BN;
    a.ncoltiles += a.seg[s].ntiles;
  }
  const int rowtiles = (a.M + BM - 1) / BM;
  const dim3 grid((unsigned)(rowtiles * a.ncoltiles)), block(NTHR);
  if (et == ET_F32) return launch_k(gemm_xw_kernel<ET_F32, BN>, grid, block, 0, stream, t, a);
  return launch_k(gemm_xw_kernel<ET_BF16, BN>, grid, block, 0, stream, t, a);
}

}  // namespace

hipError_t launch_transpose(int et, TransposeArgs a, hipStream_t stream, const LaunchTiming* t) {
  if (a.n < 1 || a.n > 4) return hipErrorInvalidValue;
  int nb = 0;
  for (int m = 0; m < a.n; ++m) {
    if (a.rows[m] < 1 || a.cols[m] < 1 || !a.src[m] || !a.dst[m]) return hipErrorInvalidValue;
    a.tile0[m] = nb;
    nb += ((a.rows[m] + 63) / 64) * ((a.cols[m] + 63) / 64);
  }
  a.tile0[a.n] = nb;
  if (et == ET_F32) return launch_k(transpose_kernel<float>, dim3(nb), dim3(256), 0, stream, t, a);
  return launch_k(transpose_kernel<uint16_t>, dim3(nb), dim3(256), 0, stream, t, a);
}

hipError_t launch_gemm(int et, GemmArgs a, hipStream_t stream, const LaunchTiming* t) {
  a.fd_ntok = make_fastdiv((uint32_t)a.Ntok);
  a.fd_d = make_fastdiv((uint32_t)a.d);
  if (a.nz < 0 || a.nz > ZR || (a.nz > 0 && (a.Wz == nullptr || a.z == nullptr))) return hipErrorInvalidValue;
  for (int s = 0; s < a.nseg; ++s) {
    GemmSeg& g = a.seg[s];
    if (g.layout == OUT_BLOCKED && (g.cg <= 0 || a.d % g.cg != 0)) return hipErrorInvalidValue;
    g.fd_cg = make_fastdiv((uint32_t)(g.cg > 0 ? g.cg : 1));
  }
  const int bn = a.tile_n ? a.tile_n : choose_tile_n(a);
  if (bn == 96) return launch_gemm_bn<96>(et, a, stream, t);
  if (bn == 128) return launch_gemm_bn<128>(et, a, stream, t);
  return hipErrorInvalidValue;
}

}  // namespace cat
