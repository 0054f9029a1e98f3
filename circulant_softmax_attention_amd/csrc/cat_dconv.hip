// cat_dconv.hip -- the 1D circulant mixing for short sequences as a direct
// product on the matrix cores (gfx950).
//
// CAT's output per head is O_h = circ(z*_h) V_h with z*_h the softmax of
// the head's logits over the N tokens (CAT: Circular-Convolutional Attention
// for Sub-Quadratic Transformers, "Key designs: circulant attention matrix
// construction"); the same page evaluates it with FFTs and remarks that at
// N = 256 the FFT route's overhead eats its O(N log N) advantage.  For
// N <= 256 this kernel forms the product directly, exactly as defined:
//
//   O[i][c] = sum_j C[i][j] V[j][c],   C[i][j] = z*[(i - j) mod N],
//
// 2 N^2 d flops per (batch, head) on MFMA, against HBM traffic of one read
// of V and one write of O: in bf16 the matrix cores keep it memory-bound at
// these lengths, and it needs no transform of either side.  (fp32 storage
// keeps the FFT path: the fp32 MFMA rate, 1/16 of bf16's, makes the direct
// product slower than the transforms there.)
//
// Workgroup: one (batch, head, half of the head's channels: 32), 256
// threads.
//  - Softmax of the head's logits in fp32 (one logit per thread, max and sum
//    over the workgroup).
//  - C is never materialised.  Its entries are the reversed, periodically
//    extended softmax line R[t] = z*[(N - t) mod N] (C[i][j] = R[j - i + N]),
//    here without the division by the sum (exp(z - max), in (0, 1], rounded
//    to bf16 (RNE); the fp32 products are divided at the end by the sum of
//    these rounded weights, so each row's weights add up to one),
//    held in LDS in 8 copies shifted by 0 .. 7 entries, so
//    that the run of 8 consecutive j values one lane feeds an MFMA is one
//    aligned 16-byte read from the copy that matches its offset.
//  - V's block [N][32] (the blocked layout with 32-channel groups) is staged
//    transposed, Vt[c][j], so a lane's run of j values for its channel is
//    one 16-byte read too.  Rows j in [N, Kp) are zero (Kp = N rounded up to
//    32), so the padded products add nothing.
//  - MFMA with A = V^T (rows: channels), B = C^T (columns: tokens i): lane
//    (lrow, lgrp) ends with O[16 tb + lrow][16 cb + 4 lgrp + v], from
//    v_mfma_f32_16x16x32_bf16 (fp32 accumulation).  Wave w takes the token
//    blocks tb = w, w + 4, .. and both 16-channel blocks.
//  - The tile goes through LDS (over the V tile) and leaves as 16-byte
//    stores of the rows' 32-channel segments.
//
// Causal CAT (CAUSAL = true).  The same page notes that a causal language
// model has to shift Z to stay causal, which costs O(N^2) ("Loss function /
// training strategy", "Limitations and outlook"): row i of circ(z) keeps
// only the tokens j <= i and is softmaxed over them,
//
//   O[i][c] = sum_{j <= i} exp(z[i - j]) V[j][c] / sum_{k <= i} exp(z[k]),
//
// exactly the O(N^2) direct product this kernel already forms.  R loses its
// periodic extension (R[t] = e[N - t] for 1 <= t <= N, zero beyond, so the
// entries j > i of each row vanish) and each row is divided by its own
// prefix sum P[i] = sum_{k <= i} e[k] (an inclusive scan in LDS) instead of
// the line's total.  e = exp(z - max over the whole line), as above; a row
// whose kept logits all lie more than about 87 below that maximum would
// underflow to 0 / 0.
#include "cat_common.hpp"
#include "cat_internal.hpp"

namespace cat {

namespace {

constexpr int DNMAX = 256;            // longest sequence of this path
constexpr int DCG = 32;               // channels per workgroup (blocked V groups)
constexpr int DTHR = 256;
constexpr int RP = 2 * DNMAX + 64;    // entries of one shifted copy of R
constexpr int RPP = RP + 8;           // copy pitch: 1168 bytes, so the 8 copies start in 8
                                      // different 16-byte bank groups
constexpr int RB = 16;                // R index offset: copy entry p holds R[p + s - RB]

constexpr int ESZ = 2;                     // bf16
constexpr int VE = 16 / ESZ;               // values per 16-byte run (and R copies)
constexpr int KS = 4 * VE;                 // j per MFMA step: 4 lane groups x VE
constexpr int VTP = (DNMAX + VE) * ESZ;    // bytes per Vt row (16-byte multiple)
constexpr int VT_BYTES = DCG * VTP;
constexpr int OP = DCG * ESZ + 16;          // O staging row pitch: 80 bytes, so the 8-byte
                                            // writes of a half-wave (16 rows x 2) hit 32
                                            // distinct bank pairs (64 bytes: 4-way)
constexpr int OS_BYTES = DNMAX * OP;        // O staging [Ip][32], padded rows
constexpr int TILE_BYTES = VT_BYTES > OS_BYTES ? VT_BYTES : OS_BYTES;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

// Block-wide max (SUM = false) or sum of one value per thread.
template <bool SUM>
__device__ __forceinline__ float block_reduce(float x, float* red) {
  auto op = [](float p, float q) { return SUM ? p + q : fmaxf(p, q); };
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = op(x, __shfl_xor(x, o, 64));
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // earlier readers of red are done
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < DTHR / 64; ++w) r = op(r, red[w]);
  return r;
}

// Inclusive prefix sum of one value per thread over the workgroup.
__device__ __forceinline__ float block_scan(float x, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(x, o, 64);
    x += lane >= o ? y : 0.f;
  }
  __syncthreads();  // earlier readers of red are done
  if (lane == 63) red[wave] = x;
  __syncthreads();
  float off = 0.f;
#pragma unroll
  for (int w = 0; w < DTHR / 64 - 1; ++w) off += w < wave ? red[w] : 0.f;
  return x + off;
}

template <bool CAUSAL>
__global__ __launch_bounds__(DTHR) void dconv_kernel(ConvArgs a) {
  using elem_t = uint16_t;  // bf16 bits
  __shared__ __attribute__((aligned(16))) char tile[TILE_BYTES];  // Vt, then the O tile
  __shared__ __attribute__((aligned(16))) elem_t rc[VE][RPP];       // shifted copies of R
  __shared__ float zs[DNMAX];
  __shared__ float red[DTHR / 64];
  __shared__ float psum[CAUSAL ? DNMAX : 1];  // causal: row normalisers P[i]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int N = a.N, ng = a.ng;
  const int q = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = q / ng, g = q - bh * ng;
  const int b = bh / a.H, h = bh - b * a.H;
  const int Kp = (N + 31) & ~31, Ip = (N + 15) & ~15;

  // The head's logits, requested first so that their latency overlaps the
  // V loads.
  const float zv = tid < N ? a.logits[(size_t)bh * N + tid] : -INFINITY;

  // ---- V block [N][32] -> Vt[c][j] (rows j >= N zero).  A unit is VE
  // consecutive tokens x VE channels: VE 16-byte loads, transposed in
  // registers, VE 16-byte LDS writes.
  {
    const elem_t* vb = reinterpret_cast<const elem_t*>(a.V) + ((size_t)bh * ng + g) * (size_t)N * DCG;
    constexpr int CPR = DCG / VE;  // 16-byte runs per token row
    const int units = (Kp / VE) * CPR;
    for (int u = tid; u < units; u += DTHR) {
      const int j0 = (u / CPR) * VE, c0 = (u % CPR) * VE;
      elem_t v[VE][VE];
#pragma unroll
      for (int r = 0; r < VE; ++r) {
        const int j = j0 + r;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (j < N) w = *reinterpret_cast<const uint4*>(vb + (size_t)j * DCG + c0);
        *reinterpret_cast<uint4*>(v[r]) = w;
      }
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        elem_t col[VE];
#pragma unroll
        for (int r = 0; r < VE; ++r) col[r] = v[r][e];
        *reinterpret_cast<uint4*>(tile + (c0 + e) * VTP + j0 * ESZ) = *reinterpret_cast<const uint4*>(col);
      }
    }
  }

  // ---- softmax of the head's logits (fp32).  The line holds exp(z - max);
  // the division by the sum is applied to the products' fp32 results, so the
  // sum's reduction runs beside the product instead of before it.
  float ev;
  {
    const float mz = block_reduce<false>(zv, red);
    // rounded to bf16 here, as the products will see it, so that the
    // normalisers below sum exactly the weights the products use (each row's
    // weights then add up to one up to fp32 rounding)
    ev = tid < N ? __uint_as_float((uint32_t)to_bf16(__expf(zv - mz)) << 16) : 0.f;
    if (tid < N) zs[tid] = ev;
  }
  __syncthreads();
  if (CAUSAL) {
    const float p = block_scan(ev, red);
    if (tid < N) psum[tid] = p;
  }
  // ---- shifted copies of R: rc[s][p] = R[p + s - RB] = z*[(N - (p + s - RB)) mod N],
  // VE entries (one 16-byte run) per item: one modulo, then the index steps
  // down by one per entry, wrapping at 0.  Causal: R[t] = e[N - t] for
  // 1 <= t <= N and zero elsewhere (no wrap).  The copy index s runs
  // fastest over the lanes, so neighbouring lanes read neighbouring logits
  // (p0 + s steps by one), free of LDS bank conflicts.
  for (int e = tid; e < VE * (RP / VE); e += DTHR) {
    const int s = e & (VE - 1), p0 = (e / VE) * VE;
    float v[VE];
    if (CAUSAL) {
#pragma unroll
      for (int u = 0; u < VE; ++u) {
        const int t = p0 + u + s - RB;
        v[u] = t >= 1 && t <= N ? zs[N - t] : 0.f;
      }
    } else {
      int idx = (N - (p0 + s - RB)) % N;
      idx += idx < 0 ? N : 0;
#pragma unroll
      for (int u = 0; u < VE; ++u) {
        v[u] = zs[idx];
        idx = idx == 0 ? N - 1 : idx - 1;
      }
    }
    *reinterpret_cast<uint4*>(&rc[s][p0]) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                       pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
  }
  __syncthreads();

  const float inv_sum = CAUSAL ? 1.f : 1.f / block_reduce<true>(ev, red);

  // ---- O^T = V^T C^T on MFMA
  constexpr int TBW = DNMAX / 16 / (DTHR / 64);  // token blocks per wave at most
  floatx4 acc[TBW][2];
#pragma unroll
  for (int t = 0; t < TBW; ++t)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[t][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int ntb = Ip / 16;
  // Lane's R run for token block t at step 0: entries p0 .. p0 + 7 of R (in
  // copy terms: copy p0 % 8, aligned start); each step moves it by KS
  // entries, a multiple of 8, so the copy stays the same.
  const elem_t* rbase[TBW];
#pragma unroll
  for (int t = 0; t < TBW; ++t) {
    const int i = 16 * (wave + 4 * t) + lrow;
    const int p0 = max(VE * lgrp - i + N + RB, 0);  // R index (VE lgrp) - i + N, plus the copy offset
                                                    // (>= 1 for every block in range)
    const int sh = p0 & (VE - 1);
    rbase[t] = &rc[sh][p0 - sh];
  }
  const char* vbase = tile + lrow * VTP + VE * lgrp * ESZ;
#pragma unroll
  for (int st = 0; st < DNMAX / KS; ++st) {
    if (st * KS >= Kp) break;
    uint4 va[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) va[cb] = *reinterpret_cast<const uint4*>(vbase + 16 * cb * VTP + st * KS * ESZ);
#pragma unroll
    for (int t = 0; t < TBW; ++t) {
      if (wave + 4 * t < ntb) {
        const uint4 cv = *reinterpret_cast<const uint4*>(rbase[t] + st * KS);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[t][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(&va[cb]),
                                                               *reinterpret_cast<const bf16x8*>(&cv),
                                                               acc[t][cb], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // every wave is done with Vt

  // ---- O tile [Ip][32] in LDS: lane holds token 16 tb + lrow, channels 16 cb + 4 lgrp + v
#pragma unroll
  for (int t = 0; t < TBW; ++t) {
    const int tb = wave + 4 * t;
    if (tb < ntb) {
      const int i = 16 * tb + lrow;
      const float inv = CAUSAL ? (i < N ? 1.f / psum[i] : 0.f) : inv_sum;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        char* dst = tile + i * OP + (16 * cb + 4 * lgrp) * ESZ;
        const floatx4 r = acc[t][cb] * inv;
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
      }
    }
  }
  __syncthreads();
  // ---- rows i < N -> O[b][i][h d + 32 g ..], 16-byte runs
  {
    constexpr int CPR = DCG * ESZ / 16;  // 16-byte runs per O row
    char* ob = reinterpret_cast<char*>(a.O) + ((size_t)b * N * a.D + (size_t)h * a.d + (size_t)g * DCG) * ESZ;
    for (int u = tid; u < N * CPR; u += DTHR) {
      const int i = u / CPR, c = u - i * CPR;
      const uint4 v = *reinterpret_cast<const uint4*>(tile + i * OP + c * 16);
      *reinterpret_cast<uint4*>(ob + (size_t)i * a.D * ESZ + c * 16) = v;
    }
  }
}

}  // namespace

hipError_t launch_dconv(int et, const ConvArgs& a, hipStream_t s, const LaunchTiming* t, bool causal) {
  if (a.N > DNMAX || a.N < 1 || a.d % DCG != 0 || a.ng != a.d / DCG || a.logits == nullptr)
    return hipErrorInvalidValue;
  const long blocks = (long)a.B * a.H * a.ng;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  if (et != ET_BF16) return hipErrorInvalidValue;  // fp32 storage keeps the FFT path
  if (causal) return launch_k(dconv_kernel<true>, dim3((unsigned)blocks), dim3(DTHR), 0, s, t, a);
  return launch_k(dconv_kernel<false>, dim3((unsigned)blocks), dim3(DTHR), 0, s, t, a);
}

}  // namespace cat
