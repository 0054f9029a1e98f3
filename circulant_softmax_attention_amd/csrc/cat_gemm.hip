// cat_gemm.hip -- the projections X . W on MFMA (gfx950).
//
// CAT projects the tokens with W_A (one score column per head) and W_V
// (CAT: Circular-Convolutional Attention for Sub-Quadratic Transformers,
// "Method details / Overall framework"); the ViT circulant attention projects
// them to Q, K and V (Vision Transformers are Circulant Attention Learners,
// "Circulant Attention: attention rebuilt with the FFT").  Both are one dense
// contraction Y = X W with X [M = B N][K = D] and W [K][ncols] as the pages
// write it.  One launch covers up to three column segments, each written in
// the layout its consumer reads.
//
// Tiling: BM x BN output tile (BM = 128 or 256, BN = 96, 128 or 192) per
// workgroup of 2 BM threads (BM / 64 x 2 waves), each wave a 64 x BN/2 block
// of 16 x 16 MFMA tiles; 256-row tiles (one workgroup per compute unit) halve
// the W tile traffic per output and are used at 192 columns.  K is
// walked in tiles of 128 bytes of an X row (64 bf16 or 32 fp32 values), i.e.
// eight 16-byte chunks; a chunk is what one lane feeds the MFMA:
//   bf16: 8 values -> v_mfma_f32_16x16x32_bf16 (fp32 accumulate)
//   fp32: 4 values -> four v_mfma_f32_16x16x4_f32
// Every lane reads the same K positions for its X row and its W column, so
// the order in which the hardware walks K inside a chunk does not matter.
//
// Staging: both operand tiles are loaded straight from global memory into
// LDS with 16-byte LDS-DMA (no register round trip), each in the layout it
// has in memory: X tiles [row][K], W tiles [K][column].  X rows are unpadded
// with the 16-byte position of chunk c in row r at c ^ ((r / 2) % 8): the 16
// rows of one fragment read (two to a 256-byte bank line) then cover all 64
// banks.  A W fragment needs the K values of one column: bf16 uses the
// transposing LDS read of gfx950 (ds_read_b64_tr_b16, 4 K values of one
// column per lane and read), fp32 one 4-byte read per value; W row k is
// rotated by rot(k) = 2 (k % 4) + 8 ((k / 8) % 2) chunks, so that the four
// rows of a lane group and the next group's four (8 rows on) fall in
// different banks.  Two LDS stages: the
// DMA of tile k + 1 is in flight while tile k is multiplied.  Rows beyond M
// and columns beyond ncols are clamped to the last valid ones (their results
// are never stored); a K tail that does not fill a tile goes through
// registers with the missing values zeroed.
//
// Score projection (1D): z = X W_A has only one column per head (at most
// 32), far too narrow for a tile of its own.  It is folded into the output
// tiles of the first segment: the first min(BM / 16, column tiles) tiles of a
// row panel share its BM / 16 16-row blocks, and the wave that owns a block
// multiplies the X fragments it already holds for the main product by W_A^T
// fragments (16 heads per MFMA block, one or two blocks).  The K tile's W_A
// rows (BK nz contiguous values) are staged in LDS with the X and W tiles and
// read transposed like a W fragment.  X is therefore read once for both
// products; z leaves head-major ([B][H][N] fp32) from registers.
#include "cat_common.hpp"
#include "cat_internal.hpp"

namespace cat {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

namespace {

constexpr int ZMAX = 32;   // score-projection columns (heads) one launch covers
constexpr int ROWB = 128;  // bytes of one X row of a K tile

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
__device__ __forceinline__ void wait_vmem_4() { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); }

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

// Rotation (in 16-byte chunks) of row k of a staged W tile, chosen per
// element type and tile width so that the 64 lanes of every fragment read
// (two transposing 8-byte reads per lane for bf16, one 4-byte read per K value
// for fp32) fall on distinct LDS banks, or on at most two where no rotation of
// this form avoids it (fp32, 96 columns).
template <int ET, int BN>
__device__ __forceinline__ int wrot(int k) {
  if constexpr (ET != ET_BF16) return 4 * ((k >> 2) & 1) + 8 * ((k >> 3) & 1);
  else if constexpr (BN == 96) return 2 * ((k >> 3) & 1);
  else if constexpr (BN == 128) return 2 * (k & 3) + 8 * ((k >> 3) & 1);
  else return 6 * (k & 3) + 6 * ((k >> 3) & 1);
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

// ZB: 16-head blocks of the score projection (0: none, at most 2).  BM: tile
// rows, 128 (256 threads, two workgroups per compute unit) or 256 (512
// threads, one workgroup per compute unit).  ZTR: bf16 W_A fragments come
// from transposing LDS reads (needs nz % 4 == 0).
template <int ET, int BN, int ZB, int BM, bool ZTR = false, bool KT = true>
__global__ __launch_bounds__(2 * BM, 256 / BM) void gemm_xw_kernel(GemmArgs a) {
  constexpr int NTHR = 2 * BM;  // 64-row wave blocks, two per row of waves
  using C = GemmCfg<ET>;
  constexpr int VE = C::VE, BK = C::BK, ESZ = C::ESZ;
  constexpr int PB = BN * ESZ;                  // bytes of one W row of the tile
  constexpr int CPRB = PB / 16;                 // 16-byte chunks per W row
  constexpr int ZT = ZB * BK * 16 * ESZ;        // W_A rows of the tile, room for 16 ZB heads
  constexpr int STAGE = BM * ROWB + BK * PB + ZT;  // one LDS stage: X rows, W rows, W_A rows
  constexpr int SMEM = 2 * STAGE;
  static_assert(ZT / 16 <= NTHR, "one W_A chunk per thread");
  constexpr int BCH = BK * CPRB / NTHR;         // W chunks per thread
  constexpr int TN = BN / 32;                   // 16-column MFMA blocks per wave
  static_assert(BCH * NTHR == BK * CPRB && TN * 32 == BN, "tile width");
  using elem_t = typename std::conditional<ET == ET_F32, float, uint16_t>::type;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int q = xcd_remap(blockIdx.x, gridDim.x);
  const int rt = q / a.ncoltiles;
  const int ctg = q - rt * a.ncoltiles;  // column tile over all segments
  int ct = ctg;
  int si = 0;
  while (si + 1 < a.nseg && ct >= a.seg[si].ntiles) {
    ct -= a.seg[si].ntiles;
    ++si;
  }
  GemmSeg sg = a.seg[si];
  const int m0 = rt * BM, n0 = ct * BN;
  // split K: slice blockIdx.y covers K positions kbase .. kbase + K - 1 and
  // writes its fp32 partial products to its own [M][ncols] slab of out
  const int kbase = (int)blockIdx.y * a.kchunk;
  const int M = a.M, K = a.K - kbase < a.kchunk ? a.K - kbase : a.kchunk, ncols = sg.ncols;
  const int ldx = a.ldx > 0 ? a.ldx : a.K;  // X row pitch (elements)
  if (blockIdx.y > 0)
    sg.out = reinterpret_cast<char*>(sg.out) + (size_t)blockIdx.y * M * ncols * (ET == ET_F32 || sg.out_f32 ? 4 : ESZ);

  // Score projection (first segment only): the first nct <= BM / 16 column
  // tiles of a row panel share its BM / 16 16-row blocks, block rb going to
  // column tile rb % nct and, inside it, to wave (rb / 4, rb % 2).  A wave
  // thus handles blocks 4 wm + wn + 2 ii, ii = 0, 1, of its own X rows.  The
  // W_A rows of each K tile ride along in the LDS stage (they are contiguous
  // in memory: BK nz values).
  const int nz = a.nz;
  const int nct = a.seg[0].ntiles < BM / 16 ? a.seg[0].ntiles : BM / 16;
  const bool zon = ZB > 0 && si == 0 && ct < nct;
  bool zrb[2];
#pragma unroll
  for (int ii = 0; ii < 2; ++ii) zrb[ii] = zon && (4 * wm + wn + 2 * ii) % nct == ct;
  const bool zwave = zrb[0] || zrb[1];

  // X tile: chunk slot s = tid + 256 i is row s / 8, 16-byte position s % 8,
  // and holds K-chunk (s % 8) ^ ((row / 2) % 8) -- the same chunk for every
  // i, since (row / 2) % 8 = (tid / 16) % 8.
  const int kch = ((tid & 7) ^ ((tid >> 4) & 7)) * VE;
  const elem_t* asrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + (NTHR / 8) * i;
    const int am = m0 + r < M ? m0 + r : M - 1;
    asrc[i] = reinterpret_cast<const elem_t*>(a.X) + (size_t)am * ldx + kbase + kch;
  }
  // W tile, K-major as W is stored: slot s = tid + 256 i is K row s / CPRB,
  // position s % CPRB, and holds column chunk (position - rot(row)) mod CPRB.
  // Columns beyond ncols are clamped to the last chunk (their results are
  // never stored).
  const elem_t* bsrc[BCH];
  int brow[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int s_ = tid + NTHR * i, k = s_ / CPRB, pos = s_ - k * CPRB;
    const int c = (pos + CPRB - wrot<ET, BN>(k) % CPRB) % CPRB;
    int col = n0 + c * VE;
    col = col + VE <= ncols ? col : ncols - VE;
    brow[i] = k;
    bsrc[i] = reinterpret_cast<const elem_t*>(sg.W) + (size_t)(kbase + k) * ncols + col;
  }
  const uint32_t lds0 = lds_addr(smem) + (uint32_t)wave * 64 * 16;
  // W_A tile: 16-byte chunk c = tid of the K tile's BK nz contiguous values
  // (8 nz chunks), read by the first 2 ZB waves; lanes past the last chunk
  // repeat it (into the padding of the stage's W_A room).
  const int zchunks = ZB > 0 ? 8 * nz : 0;
  const bool zdma = zon && wave < 2 * ZB;
  const char* zsrc = reinterpret_cast<const char*>(a.Wz) + 16 * (size_t)(tid < zchunks ? tid : zchunks - 1);

  // K order: the workgroups that share a W tile (one column tile, the
  // neighbouring row panels on an XCD) or an X tile (one row panel) start at
  // different K tiles, so that at any moment they ask for different lines.
  const int nk = (K + BK - 1) / BK;
  const int koff = rt % nk;
  auto kmap = [&](int kt) { return kt + koff < nk ? kt + koff : kt + koff - nk; };

  // Stage the kt-th K tile (in this workgroup's order) into LDS stage st.
  auto issue = [&](int kt, int st) {
    const int k0 = kmap(kt) * BK;
    if (!KT || k0 + BK <= K) {
      const uint32_t base = lds0 + (uint32_t)(st * STAGE);
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_dma16(asrc[i] + k0, base + i * NTHR * 16);
#pragma unroll
      for (int i = 0; i < BCH; ++i) lds_dma16(bsrc[i] + (size_t)k0 * ncols, base + BM * ROWB + i * NTHR * 16);
      if (ZB > 0 && zdma) lds_dma16(zsrc + (size_t)k0 * nz * ESZ, base + BM * ROWB + BK * PB);
    } else {
      // K tail: X chunks and W rows at or beyond K are zero
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
        const bool okb = k0 + brow[i] < K;
        const uint4 v = *reinterpret_cast<const uint4*>(bsrc[i] + (okb ? (size_t)k0 * ncols : 0));
        vb[i] = okb ? v : make_uint4(0, 0, 0, 0);
      }
      uint4* dst = reinterpret_cast<uint4*>(smem + st * STAGE) + tid;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i * NTHR] = va[i];
#pragma unroll
      for (int i = 0; i < BCH; ++i) dst[BM * 8 + i * NTHR] = vb[i];
      if (ZB > 0 && zon && tid < ZT / 16) {  // W_A values of rows at or beyond K (and the padding) are zero
        const elem_t* wz = reinterpret_cast<const elem_t*>(a.Wz) + (size_t)k0 * nz;
        elem_t e[VE];
#pragma unroll
        for (int j = 0; j < VE; ++j) {
          const int f = VE * tid + j;
          e[j] = tid < zchunks && k0 + f / nz < K ? wz[f] : elem_t(0);
        }
        reinterpret_cast<uint4*>(smem + st * STAGE + BM * ROWB + BK * PB)[tid] = *reinterpret_cast<const uint4*>(e);
      }
    }
  };

  // Whole-tile kernels (512 threads): the DMA slots of wave + 4 (thread
  // tid + 256) as well, for waves 0-3, which issue both (see step)
  const elem_t* bsrc2[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int s_ = tid + 256 + NTHR * i, k = s_ / CPRB, pos = s_ - k * CPRB;
    const int c = (pos + CPRB - wrot<ET, BN>(k) % CPRB) % CPRB;
    int col = n0 + c * VE;
    col = col + VE <= ncols ? col : ncols - VE;
    bsrc2[i] = reinterpret_cast<const elem_t*>(sg.W) + (size_t)(kbase + k) * ncols + col;
  }
  const elem_t* asrc2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ((tid + 256) >> 3) + (NTHR / 8) * i;
    const int am = m0 + r < M ? m0 + r : M - 1;
    asrc2[i] = reinterpret_cast<const elem_t*>(a.X) + (size_t)am * ldx + kbase + kch;
  }
  auto issue2 = [&](int kt, int st) {
    const int k0 = kmap(kt) * BK;
    const uint32_t base = lds0 + (uint32_t)(st * STAGE);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lds_dma16(asrc[i] + k0, base + i * NTHR * 16);
      lds_dma16(asrc2[i] + k0, base + 4096 + i * NTHR * 16);
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      lds_dma16(bsrc[i] + (size_t)k0 * ncols, base + BM * ROWB + i * NTHR * 16);
      lds_dma16(bsrc2[i] + (size_t)k0 * ncols, base + 4096 + BM * ROWB + i * NTHR * 16);
    }
    if (ZB > 0 && zdma) lds_dma16(zsrc + (size_t)k0 * nz * ESZ, base + BM * ROWB + BK * PB);
  };
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int sw = (lrow >> 1) & 7;  // (row / 2) % 8 of every X fragment row this lane reads
  floatx4 acc[4][TN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Fragment of 16 columns (col0 ..) x one K step of a K-major tile (row
  // pitch `pitch` bytes, `cpr` chunks, rows rotated by rot(k) chunks) for
  // this lane: column col0 + lrow, the K values of group lgrp.  bf16: two
  // transposing LDS reads, each giving 4 consecutive K values of the lane's
  // column (the 16 lanes of a group address 4 rows x 4 column quads); fp32:
  // one 4-byte read per K value.
  auto kfrag = [&](const char* tile, int pitch, int cpr, int col0, int kc) -> uint4 {
    if constexpr (ET == ET_BF16) {
      typedef short v4s __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4s lds_v4s;
      const int c = col0 / 8 + ((lrow & 3) >> 1);
      uint2 part[2];
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const int k = kc * 32 + 8 * lgrp + 4 * hlf + (lrow >> 2);
        const int pos = (c + wrot<ET, BN>(k)) % cpr;
        const char* ptr = tile + k * pitch + pos * 16 + 8 * (lrow & 1);
        const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4s*)(const __attribute__((address_space(3))) char*)ptr);
        part[hlf] = *reinterpret_cast<const uint2*>(&r);
      }
      return make_uint4(part[0].x, part[0].y, part[1].x, part[1].y);
    } else {
      float f[4];
      const int col = col0 + lrow;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = kc * 16 + 4 * lgrp + u;
        const int pos = (col / 4 + wrot<ET, BN>(k)) % cpr;
        f[u] = *reinterpret_cast<const float*>(tile + k * pitch + pos * 16 + 4 * (col & 3));
      }
      return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
  };

  // Fragments of K-chunk kc (0 or 1) of the tile in stage st.
  auto read_frags = [&](int st, int kc, uint4 (&af)[4], uint4 (&bf)[TN]) {
    const char* sa = smem + st * STAGE + (wm * 64 + lrow) * ROWB;
    const char* sb = smem + st * STAGE + BM * ROWB;
    const int pos = ((kc * 4 + lgrp) ^ sw) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const uint4*>(sa + 16 * i * ROWB + pos);
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[j] = kfrag(sb, PB, CPRB, wn * (BN / 2) + 16 * j, kc);
  };
  // W fragment as the MFMA's A operand, X fragment as B: the 16 x 16 result
  // is Y^T, so each lane ends with 4 consecutive channels of one token (see
  // the stores below)
  auto mma = [&](const uint4 (&af)[4], const uint4 (&bf)[TN]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma_chunk<ET>(bf[j], af[i], acc[i][j]);
  };

  // W_A^T fragment of K step kc for heads 16 zb ..: lane (lrow, lgrp) holds
  // head 16 zb + lrow at the K positions of its X fragments, read from the
  // stage's W_A rows [BK][nz] (row pitch nz values).  bf16 with nz % 4 == 0:
  // two transposing reads, the lanes of a group addressing 4 rows x 4 head
  // quads exactly as for a W fragment (heads past nz read the next row's
  // values or the zero padding; their results are never stored); otherwise
  // one read per K value.  Heads past nz are clamped in the per-value reads.
  constexpr int ZA = ZB > 0 ? ZB : 1;  // register arrays need a size
  const int zp = nz * ESZ;             // bytes per W_A row
  auto zfrag = [&](int st, int zb, int kc) -> uint4 {
    const char* zt = smem + st * STAGE + BM * ROWB + BK * PB;
    if constexpr (ET == ET_BF16) {
      if constexpr (ZTR) {
        typedef short v4s __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) v4s lds_v4s;
        uint2 part[2];
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          const int k = kc * 32 + 8 * lgrp + 4 * hlf + (lrow >> 2);
          const char* ptr = zt + k * zp + 32 * zb + 8 * (lrow & 3);
          const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4s*)(const __attribute__((address_space(3))) char*)ptr);
          part[hlf] = *reinterpret_cast<const uint2*>(&r);
        }
        return make_uint4(part[0].x, part[0].y, part[1].x, part[1].y);
      } else {
        const int h0 = 16 * zb + lrow, h = h0 < nz ? h0 : nz - 1;
        uint32_t w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int k = kc * 32 + 8 * lgrp + 2 * u;
          const uint32_t lo = *reinterpret_cast<const uint16_t*>(zt + k * zp + 2 * h);
          const uint32_t hi = *reinterpret_cast<const uint16_t*>(zt + (k + 1) * zp + 2 * h);
          w[u] = lo | (hi << 16);
        }
        return make_uint4(w[0], w[1], w[2], w[3]);
      }
    } else {
      const int h0 = 16 * zb + lrow, h = h0 < nz ? h0 : nz - 1;
      uint32_t w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = *reinterpret_cast<const uint32_t*>(zt + (kc * 16 + 4 * lgrp + u) * zp + 4 * h);
      return make_uint4(w[0], w[1], w[2], w[3]);
    }
  };
  floatx4 zacc[2][ZA];  // [ii][zb]
#pragma unroll
  for (int ii = 0; ii < 2; ++ii)
#pragma unroll
    for (int zb = 0; zb < ZA; ++zb) zacc[ii][zb] = floatx4{0.f, 0.f, 0.f, 0.f};
  // The X fragment of block ii is af[wn + 2 ii]; wn is uniform, so the two
  // cases are separate branches rather than per-lane selects.
  auto zmma_wn = [&](int kc, const uint4 (&af)[4], int st, auto wn_tag) {
    constexpr int WN = decltype(wn_tag)::value;
#pragma unroll
    for (int zb = 0; zb < ZB; ++zb) {
      const uint4 wf = zfrag(st, zb, kc);
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
        if (zrb[ii]) zacc[ii][zb] = mfma_chunk<ET>(wf, af[WN + 2 * ii], zacc[ii][zb]);
    }
  };
  auto zmma = [&](int kc, const uint4 (&af)[4], int st) {
    if (ZB == 0 || !zwave) return;
    if (wn)
      zmma_wn(kc, af, st, std::integral_constant<int, 1>{});
    else
      zmma_wn(kc, af, st, std::integral_constant<int, 0>{});
  };

  // Tile kt lives in stage kt % 2.  At the top of step kt every wave has its
  // own DMA of tile kt complete and, after the barrier, all of them have
  // finished multiplying tile kt - 1, whose stage then receives tile kt + 1,
  // whose DMA thus runs under the MFMAs of tile kt.  The loop is unrolled by
  // two so that stage indices are compile-time constants.
  const bool warm = BN != 192 && a.warm;
  issue(0, 0);
  // L2 warm-up, where a row panel is read by many column tiles: those tiles
  // (consecutive workgroups on one XCD) together touch every 64-byte sector
  // of the panel's X rows once, right after the first tile's DMA, so that
  // the DMAs of the later K tiles hit L2 rather than all missing at once.
  // Four loads per thread cover panels of up to 4 x 256 x (column tiles)
  // sectors; step 0 waits for the first tile only (the warm-up loads were
  // issued after it), and the values feed a test that never passes.
  constexpr int WARM = 4;
  uint32_t wv[WARM] = {0u, 0u, 0u, 0u};
  if (warm) {
    const int rows = M - m0 < BM ? M - m0 : BM;
    const uint32_t spr = (uint32_t)(K * ESZ + 63) / 64;  // sectors per row
    const uint32_t nsec = (uint32_t)rows * spr;
    const char* xb = reinterpret_cast<const char*>(a.X) + ((size_t)m0 * ldx + kbase) * ESZ;
#pragma unroll
    for (int u = 0; u < WARM; ++u) {
      uint32_t sidx = (uint32_t)ctg + (uint32_t)a.ncoltiles * (uint32_t)(tid + NTHR * u);
      sidx = sidx < nsec ? sidx : nsec - 1;
      const uint32_t r = sidx / spr, c = sidx - r * spr;
      wv[u] = *reinterpret_cast<const uint32_t*>(xb + (size_t)r * ldx * ESZ + (size_t)c * 64);
    }
  }
  uint4 af[4], bf[TN];
  auto step = [&](int kt, auto parity) {
    constexpr int st = decltype(parity)::value;
    if (kt == 0 && warm)
      wait_vmem_4();
    else
      wait_vmem_all();
    __syncthreads();
    if constexpr (!KT) {
      // Waves 0-3 issue the next tile's DMA for themselves and for waves
      // 4-7, which go straight to their products.  A wave waits at a DMA
      // instruction until the address unit takes it, and the unit takes a
      // compute unit's requests one by one; with every wave issuing its own
      // share, the waves queued last started their products up to 1 us late.
      // (The kernels with a K tail keep every wave issuing its own share.)
      static_assert(NTHR == 512, "whole-tile kernels are the 256-row, 512-thread ones");
      if (kt + 1 < nk && wave < 4) issue2(kt + 1, st ^ 1);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        read_frags(st, kc, af, bf);
        mma(af, bf);
        zmma(kc, af, st);
      }
    } else {
      if (kt + 1 < nk) issue(kt + 1, st ^ 1);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        read_frags(st, kc, af, bf);
        mma(af, bf);
        zmma(kc, af, st);
      }
    }
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>{});
  }
  if (warm && ((wv[0] ^ wv[1]) + (wv[2] ^ wv[3])) == 0x9E3779B9u && M < 0)  // keeps the warm-up loads
    reinterpret_cast<float*>(sg.out)[0] = 0.f;

  // Result layout (16 x 16 MFMA, A = W rows, B = X rows): lane (lrow, lgrp)
  // holds Y[token][channel] for token = tile row base + lrow and the four
  // channels 4 lgrp + v, v = 0..3, of each 16-channel block.
  // z [B][nz][Ntok] fp32: lane holds token lrow of its row block and heads
  // 16 zb + 4 lgrp + v; the 16 lanes of a head cover 16 consecutive tokens
  if (ZB > 0 && zwave) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int token = m0 + wm * 64 + 16 * (wn + 2 * ii) + lrow;
      if (zrb[ii] && token < M) {
        const uint32_t b = fastdiv((uint32_t)token, a.fd_ntok);
        const uint32_t tok = (uint32_t)token - b * (uint32_t)a.Ntok;
#pragma unroll
        for (int zb = 0; zb < ZB; ++zb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int head = 16 * zb + 4 * lgrp + v;
            if (head < nz) a.z[((size_t)b * nz + head) * a.Ntok + tok] = zacc[ii][zb][v];
          }
      }
    }
  }
  const bool f32out = ET == ET_F32 || sg.out_f32;
  // Staged epilogue: when every aligned group of 16 bytes of channels is
  // contiguous in the output, the tile goes through LDS (free once every wave
  // is done with the last K tile) and leaves in 16-byte stores whose lanes
  // cover whole row segments -- far faster for the memory system than the
  // 8-byte, 16-rows-apart stores the register layout gives.
  const int vo = f32out ? 4 : 8;  // channels per 16 bytes of output
  constexpr bool FIT4 = BM * BN * 4 <= SMEM;  // an fp32 tile fits the LDS
  const bool staged = (!f32out || FIT4) && ((sg.layout == OUT_ROWMAJOR && ncols % vo == 0) ||
                                            (sg.layout == OUT_BLOCKED && sg.cg % vo == 0 && a.d % vo == 0));
  if (staged) {
    auto stage_out = [&](auto osz_tag) {
      constexpr int OSZ = decltype(osz_tag)::value;
      constexpr int VO = 16 / OSZ;
      constexpr int CPR = BN * OSZ / 16;  // 16-byte chunks per tile row
      constexpr int PITCH = BM * (BN * OSZ + 16) <= SMEM ? BN * OSZ + 16 : BN * OSZ;
      constexpr int PER = BM * CPR / NTHR;
      static_assert(PER * NTHR == BM * CPR && BM * PITCH <= SMEM, "staged tile");
      __syncthreads();  // every wave is done reading the last K tile
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const floatx4 v = acc[i][j];
          char* dst = smem + (wm * 64 + 16 * i + lrow) * PITCH + (wn * (BN / 2) + 16 * j + 4 * lgrp) * OSZ;
          if constexpr (OSZ == 4) *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
          else *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int c = tid + NTHR * u;
        const int row = c / CPR, cc = c - row * CPR;
        const int token = m0 + row, ch = n0 + cc * VO;
        if (token < M && ch < ncols) {
          const uint4 v = *reinterpret_cast<const uint4*>(smem + row * PITCH + cc * 16);
          *reinterpret_cast<uint4*>(reinterpret_cast<char*>(sg.out) + out_index(sg, a, token, ch) * OSZ) = v;
        }
      }
    };
    if constexpr (FIT4) {
      if (f32out) stage_out(std::integral_constant<int, 4>{});
      else stage_out(std::integral_constant<int, 2>{});
    } else {
      stage_out(std::integral_constant<int, 2>{});
    }
    return;
  }
  // (192-wide tiles are launched only where the staged path applies)
  if constexpr (BN != 192) {
  // Otherwise straight from registers: 8 (bf16) or 16 (fp32) bytes per lane,
  // the 16 lanes of a channel block covering 16 consecutive tokens.
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
}

// Output tile width: 192, 128 or 96 columns.  Two 128-row workgroups fit a
// compute unit, so the grid runs in rounds of 2 x CUs workgroups; the
// estimated time is rounds x (BN + 48) (a tile costs its columns plus a fixed
// part), and the cheapest width is taken.  192-column tiles are for 2-byte
// operands and 2-byte outputs that take the staged epilogue only (the LDS
// holds two stages of an fp32 W tile of that width, or an fp32 output tile,
// only barely or not), and for at most 16 score-projection heads (more would
// not fit the registers).
bool wide_ok(int et, const GemmArgs& a) {
  bool ok = et != ET_F32 && a.nz <= 16;
  for (int s = 0; s < a.nseg; ++s) {
    const GemmSeg& g = a.seg[s];
    ok = ok && !g.out_f32 &&
         ((g.layout == OUT_ROWMAJOR && g.ncols % 8 == 0) || (g.layout == OUT_BLOCKED && g.cg % 8 == 0 && a.d % 8 == 0));
  }
  return ok;
}

long col_tiles(const GemmArgs& a, int bn) {
  long t = 0;
  for (int s = 0; s < a.nseg; ++s) t += (a.seg[s].ncols + bn - 1) / bn;
  return t;
}

int choose_tile_n(int et, const GemmArgs& a) {
  const long cus = a.num_cu > 0 ? a.num_cu : 256;
  const long rowtiles = (a.M + 127) / 128;
  const long slots = 2 * cus;
  int best = 128;
  long best_cost = -1;
  const bool stage2 = wide_ok(et, a);
  for (int bn : {192, 128, 96}) {
    if (bn == 192 && !stage2) continue;
    const long tiles = rowtiles * col_tiles(a, bn);
    const long cost = ((tiles + slots - 1) / slots) * (bn + 48);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = bn;
    }
  }
  return best;
}

// 256-row tiles (one 512-thread workgroup per compute unit) halve the W tile
// traffic per output; they exist for 2-byte operands at 128 or 192 columns
// and are taken at 192 columns (at 128 they measured slower) when they need
// no more rounds than 128-row tiles and give every compute unit a tile.
bool tall_ok(int et, int bn) { return et != ET_F32 && (bn == 128 || bn == 192); }

int choose_tile_m(int et, const GemmArgs& a, int bn) {
  if (!tall_ok(et, bn) || bn != 192) return 128;
  const long cus = a.num_cu > 0 ? a.num_cu : 256;
  const long ct = col_tiles(a, bn);
  const long t128 = (a.M + 127) / 128 * ct, t256 = (a.M + 255) / 256 * ct;
  const long r128 = (t128 + 2 * cus - 1) / (2 * cus), r256 = (t256 + cus - 1) / cus;
  return t256 >= cus && r256 <= r128 ? 256 : 128;
}

template <int BN, int BM>
hipError_t launch_gemm_bn(int et, GemmArgs& a, hipStream_t stream, const LaunchTiming* t) {
  a.ncoltiles = 0;
  for (int s = 0; s < a.nseg; ++s) {
    a.seg[s].ntiles = (a.seg[s].ncols + BN - 1) / BN;
    a.ncoltiles += a.seg[s].ntiles;
  }
  const int rowtiles = (a.M + BM - 1) / BM;
  const dim3 grid((unsigned)(rowtiles * a.ncoltiles), (unsigned)a.ksplit), block(2 * BM);
  a.warm = a.ncoltiles > 8 ? 1 : 0;  // the L2 warm-up measured faster at 9 column tiles, slower at 4 and 8
  const int zb = (a.nz + 15) / 16;
  const bool tr = a.nz % 4 == 0;
  if (et == ET_F32) {
    if constexpr (BN == 192 || BM == 256) {  // 2-byte operands only
      return hipErrorInvalidValue;
    } else {
      if (zb == 0) return launch_k(gemm_xw_kernel<ET_F32, BN, 0, BM>, grid, block, 0, stream, t, a);
      if (zb == 1) return launch_k(gemm_xw_kernel<ET_F32, BN, 1, BM>, grid, block, 0, stream, t, a);
      return launch_k(gemm_xw_kernel<ET_F32, BN, 2, BM>, grid, block, 0, stream, t, a);
    }
  }
  // KT = false: every K slice is whole K tiles, so the kernel carries no
  // tail path (and none of the registers it would hold)
  auto bf16 = [&](auto kt_tag) -> hipError_t {
    constexpr bool KT = decltype(kt_tag)::value;
    if (zb == 0) return launch_k(gemm_xw_kernel<ET_BF16, BN, 0, BM, false, KT>, grid, block, 0, stream, t, a);
    // 128 x 192 tiles never carry the score projection, 256 x 192 ones at
    // most 16 heads
    if constexpr (BN == 192 && BM == 128) {
      return hipErrorInvalidValue;
    } else {
      if (zb == 1)
        return tr ? launch_k(gemm_xw_kernel<ET_BF16, BN, 1, BM, true, KT>, grid, block, 0, stream, t, a)
                  : launch_k(gemm_xw_kernel<ET_BF16, BN, 1, BM, false, KT>, grid, block, 0, stream, t, a);
      if constexpr (BN == 192) {
        return hipErrorInvalidValue;
      } else {
        return tr ? launch_k(gemm_xw_kernel<ET_BF16, BN, 2, BM, true, KT>, grid, block, 0, stream, t, a)
                  : launch_k(gemm_xw_kernel<ET_BF16, BN, 2, BM, false, KT>, grid, block, 0, stream, t, a);
      }
    }
  };
  if constexpr (BM == 256) {
    if (a.K % 64 == 0) return bf16(std::false_type{});
  }
  return bf16(std::true_type{});
}

}  // namespace

hipError_t launch_gemm(int et, GemmArgs a, hipStream_t stream, const LaunchTiming* t) {
  a.fd_ntok = make_fastdiv((uint32_t)a.Ntok);
  a.fd_d = make_fastdiv((uint32_t)a.d);
  a.fd_nz = make_fastdiv((uint32_t)(a.nz > 0 ? a.nz : 1));
  if (a.nz < 0 || a.nz > ZMAX || (a.nz > 0 && (a.Wz == nullptr || a.z == nullptr))) return hipErrorInvalidValue;
  if (a.ldx != 0 && (a.ldx < a.K || a.ldx % (et == ET_F32 ? 4 : 8) != 0)) return hipErrorInvalidValue;
  // split K: slices of kchunk (a multiple of the K tile) K positions, each
  // writing fp32 row-major partial products; no score projection
  if (a.ksplit <= 1) {
    a.ksplit = 1;
    a.kchunk = a.K;
  } else {
    const int bk = et == ET_F32 ? 32 : 64;
    if (a.nz != 0 || a.kchunk < bk || a.kchunk % bk != 0 || (long)(a.ksplit - 1) * a.kchunk >= a.K ||
        (long)a.ksplit * a.kchunk < a.K || a.ksplit > 65535)
      return hipErrorInvalidValue;
    for (int s = 0; s < a.nseg; ++s)
      if (a.seg[s].layout != OUT_ROWMAJOR || !a.seg[s].out_f32) return hipErrorInvalidValue;
  }
  for (int s = 0; s < a.nseg; ++s)
    if (a.seg[s].ncols % (et == ET_F32 ? 4 : 8) != 0) return hipErrorInvalidValue;  // whole 16-byte column chunks
  for (int s = 0; s < a.nseg; ++s) {
    GemmSeg& g = a.seg[s];
    if (g.layout == OUT_BLOCKED && (g.cg <= 0 || a.d % g.cg != 0)) return hipErrorInvalidValue;
    g.fd_cg = make_fastdiv((uint32_t)(g.cg > 0 ? g.cg : 1));
  }
  int bn = a.tile_n ? a.tile_n : choose_tile_n(et, a);
  if (bn == 192 && !wide_ok(et, a)) bn = choose_tile_n(et, a);
  int bm = a.tile_m ? a.tile_m : choose_tile_m(et, a, bn);
  if (bm == 256 && !tall_ok(et, bn)) bm = 128;
  // with W_A rows in every stage, two 128 x 192 workgroups no longer fit a
  // compute unit's LDS
  if (bn == 192 && bm == 128 && a.nz > 0) bn = 128;
  if (bm == 256) {
    if (bn == 128) return launch_gemm_bn<128, 256>(et, a, stream, t);
    if (bn == 192) return launch_gemm_bn<192, 256>(et, a, stream, t);
    return hipErrorInvalidValue;
  }
  if (bn == 96) return launch_gemm_bn<96, 128>(et, a, stream, t);
  if (bn == 128) return launch_gemm_bn<128, 128>(et, a, stream, t);
  if (bn == 192) return launch_gemm_bn<192, 128>(et, a, stream, t);
  return hipErrorInvalidValue;
}

}  // namespace cat
