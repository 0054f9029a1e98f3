// cat_internal.hpp -- argument blocks and launchers shared by the C-ABI layer
// and the kernel translation units (host-visible, no device code).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/cat.h"

namespace cat {

enum ElemType : int { ET_F32 = 0, ET_BF16 = 1 };

// Optional per-launch timing: two events that the kernel's own dispatch
// stamps at its start and its end (hipExtLaunchKernel), so no marker packet
// sits between the kernels of a call.
struct LaunchTiming {
  hipEvent_t start, stop;
};

template <typename K, typename... Args>
inline hipError_t launch_k(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, const LaunchTiming* t,
                           Args... args) {
  if (t)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, t->start, t->stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  return hipGetLastError();
}

// Output index maps of the projection GEMM.  Row m = b * Ntok + tok.
//   ROWMAJOR: out[m * ncols + n]
//   BLOCKED : channel n of head h = n / d lands in group g = (n % d) / cg:
//             out[(((b * H + h) * (d / cg) + g) * Ntok + tok) * cg + n % cg]
//             -- every group is one contiguous [Ntok][cg] block, the unit a
//             transform workgroup reads.
//   HEADMAJOR: out[(b * ncols + n) * Ntok + tok] (score logits, [B][H][N])
enum OutLayout : int { OUT_ROWMAJOR = 0, OUT_BLOCKED = 1, OUT_HEADMAJOR = 2 };

// Division by a runtime-invariant divisor as a multiply-high and a shift
// (round-up magic number; exact for 0 <= x < 2^31 and 1 <= div < 2^31).
struct FastDiv {
  uint32_t div, mul, shr;
};
inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.div = d;
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;
  f.shr = s;
  f.mul = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1);
  return f;
}
__host__ __device__ inline uint32_t fastdiv(uint32_t x, const FastDiv& f) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t t = __umulhi(x, f.mul);
#else
  const uint32_t t = (uint32_t)(((uint64_t)x * f.mul) >> 32);
#endif
  return (t + x) >> f.shr;
}

struct GemmSeg {
  const void* W;  // [K][ncols] row-major, same element type as X; ncols a multiple of 16 bytes
  void* out;
  int ncols;
  int out_f32;  // 1: fp32 output; 0: the input element type
  int layout;   // OutLayout
  int cg;       // channels per group (BLOCKED)
  // filled by the launcher
  int ntiles;
  FastDiv fd_cg;
};

struct GemmArgs {
  const void* X;  // [M][K] row-major, rows ldx elements apart
  int M, K;
  int ldx;  // X row pitch in elements, a multiple of 16 bytes (0: K)
  // split K (ksplit > 1): slice s takes K positions s kchunk .. and writes
  // segment outputs (row-major fp32 only) at out + s M ncols; no score
  // projection.  ksplit <= 1: one slice.
  int ksplit, kchunk;
  int Ntok, H, d;
  int nseg;
  // optional score projection (1D): z [M / Ntok][nz][Ntok] fp32 = X . Wz,
  // Wz = W_A [K][nz]; nz = 0 disables it, at most 32
  const void* Wz;
  float* z;
  int nz;
  int tile_n;  // output tile width (96, 128 or 192); 0 lets the launcher choose
  int tile_m;  // output tile rows (128 or 256); 0 lets the launcher choose
  FastDiv fd_nz;  // filled by the launcher
  int num_cu;  // compute units of the device (0: assume 256)
  // filled by the launcher
  int ncoltiles;
  int warm;  // 1: the GEMM warms L2 with each row panel's X first
  FastDiv fd_ntok, fd_d;
  GemmSeg seg[3];
};

// Launch Y_s = X . W_s for every segment s (and z when nz > 0); returns
// hipSuccess or the launch error.
hipError_t launch_gemm(int et, GemmArgs args, hipStream_t stream, const LaunchTiming* t = nullptr);

// Softmax + spectrum of one line per (batch, head).
//   mode 0: input logits [BH][N] (fp32, spatial, not yet scaled)
//   mode 1: input partial spectra [BH][ngrp][L] (complex fp32, 2D scores),
//           summed and inverse-transformed to the logits first
// The logits are multiplied by `scale`, softmaxed over the N valid positions
// (optionally written to `probs` [BH][N]), laid on the length-L transform
// line (periodically extended when L > N in 1D), multiplied by 1/L and
// forward transformed:  spec[bh][k1 + L1 k2].
struct SpecArgs {
  const float* logits;
  const float2* partial;
  int ngrp;
  float2* spec;
  float* probs;
  const float2* tw;  // 1D inter-pass twiddles (may be null for 2D)
  int BH, N;
  float scale;
  int G, log2G;  // lines per workgroup
  int transpose;  // 2D only: write spec[bh][k2 + L2 k1] (k2 contiguous) instead of k1 + L1 k2
};

// Fused forward transform . Hadamard . inverse transform of one group of
// 2G channels (G complex lines) of one (batch, head):
//   O[b][p][h d + g 2G + c] = IFFT(spec[bh] . FFT(V line))[p]   for p < N
struct ConvArgs {
  const void* V;      // BLOCKED [B][H][ng][N][2G], element type et
  const float2* spec; // [BH][L]
  const float* logits;  // matrix-core and direct convs: [BH][N] fp32 logits whose
                        // softmax (and its spectrum) the conv computes itself (spec unused)
  const float2* tw;   // 1D inter-pass twiddles (null for 2D; unused by the matrix-core conv)
  const void* mtab;   // 1D matrix-core conv: its per-lane constant table (mconv_table_halfs fp16 values)
  void* O;            // [B][N][D], element type et
  int B, H, D, N, d;
  int G, log2G, ng;
};

// 2D scores: for each (bh, group of pairs) accumulate
//   sum_pairs FFT2(q pair) . conj(FFT2(k pair))   into partial[bh][grp][L]
struct ScoreArgs {
  const void* Q;  // BLOCKED [BH][npair / (cg / 2)][N][cg], element type et
  const void* K;
  float2* partial;  // [BH][ngrp][L] complex
  int BH, N, npair, ngrp, ppg;
  const float2* tw;  // 1D inter-pass twiddles (null for 2D)
  int et, cg;        // ET_F32 (2D: fp32, cg = 2) or ET_BF16 (1D only); cg even, (cg / 2) | npair
};

struct RelayoutArgs {
  const void* src;  // [B][N][D] row-major
  void* dst;        // BLOCKED
  int src_et, dst_f32;
  int B, N, D, H, d, cg;
};

// Transform geometry chosen for a problem.
struct LineGeom {
  int L1, L2;  // L = L1 * L2
  int twiddled;  // 1D (inter-pass twiddles) vs 2D grid
};

// Supported geometries.  1D: powers of two 1..4096; 2D: a fixed list of grids.
bool geom_supported(const LineGeom& g);
// LDS bytes of one transform line and the threads per line.
size_t line_lds_bytes(const LineGeom& g);
int line_threads(const LineGeom& g);
// Threads per DFT of a geometry (2 for split grids, whose lines take one
// workgroup each), 0 if unsupported.
int line_split(const LineGeom& g);
// LDS bytes of a spectrum workgroup of G lines (lines, reduction scratch).
size_t spectrum_lds_bytes(const LineGeom& g, int G);

// mode 0: softmax spectrum from logits; 1 (2D): from summed score partials;
// 2 (1D): the logits gradient of the mixing backward into a.probs.
hipError_t launch_spectrum(const LineGeom& g, int mode, const SpecArgs& a, hipStream_t s,
                           const LaunchTiming* t = nullptr);
hipError_t launch_conv(const LineGeom& g, int et, const ConvArgs& a, hipStream_t s, const LaunchTiming* t = nullptr);
// 1D FFT-convolution for L = 1024 with the radix-32 passes on the matrix
// cores (bf16 storage), softmax spectrum of a.logits [BH][N] included (a.spec
// unused): V BLOCKED with 8-channel groups (a.ng = d / 8), N <= 1024,
// d % 16 == 0, a.logits and a.mtab set.
hipError_t launch_mconv(const ConvArgs& a, hipStream_t s, const LaunchTiming* t = nullptr);
// The matrix-core conv's constant table: [q][lane][slot s] fp16, q = 0..7:
// F re, F im for x = 0 (q = 0, 1) and x = 1 (q = 2, 3), then the twiddle
// W^(j k) / 32 re, im for x = 0 (q = 4, 5) and x = 1 (q = 6, 7), with
// j = lane % 16 + 16 x, k = 4 (lane / 16) + s % 4 + 16 (s / 4),
// F[j][k] = exp(-2 pi i (j k mod 32) / 32), W = exp(-2 pi i / 1024).
constexpr size_t mconv_table_halfs() { return 8 * 64 * 8; }
// 1D circulant mixing for N <= 256 as the direct product circ(z*) V on the
// matrix cores, softmax of a.logits [BH][N] included: bf16 storage only
// (et == ET_BF16), V BLOCKED with 32-channel groups (a.ng = d / 32),
// d % 32 == 0; a.spec and a.tw unused.  causal: each row i keeps only the
// tokens j <= i and is normalised over them (causal CAT).
hipError_t launch_dconv(int et, const ConvArgs& a, hipStream_t s, const LaunchTiming* t = nullptr,
                        bool causal = false);
hipError_t launch_score_partial(const LineGeom& g, const ScoreArgs& a, hipStream_t s,
                                const LaunchTiming* t = nullptr);
// The same partials on the 96 x 96 grid (cat_score96.hip): fp32 pair lines
// (et == ET_F32, cg == 2), a.N == 9216, a.ngrp == ceil(npair / ppg); a.tw
// unused.  launch_score_partial routes the 96 x 96 grid here.
hipError_t launch_score96(const ScoreArgs& a, hipStream_t s, const LaunchTiming* t = nullptr);
// The scores-mode spectrum (logits = Re IFFT2 of the summed partials times
// a.scale, softmax, FFT2 / N) on the 96 x 96 grid (cat_score96.hip): a.N ==
// 9216, a.partial with a.ngrp partials per (batch, head); a.logits, a.tw
// and a.G unused.  launch_spectrum routes mode 1 on the 96 x 96 grid here.
hipError_t launch_spec96(const SpecArgs& a, hipStream_t s, const LaunchTiming* t = nullptr);
// Projection-gradient helpers of the CAT backward (cat_backward.hip), storage
// dtype et: dst [C][ldd] = src [R][C]^T with columns R .. ldd - 1 zero;
// P [B N][D + Hp] = [dV | dz token-major | 0] (Hp >= H; D and Hp multiples
// of 8).
hipError_t launch_transpose(int et, const void* src, void* dst, int R, int C, int ldd, hipStream_t s,
                            const LaunchTiming* t = nullptr);
hipError_t launch_pack_grads(int et, const void* dV, const float* dz, void* P, int B, int N, int D, int H, int Hp,
                             hipStream_t s, const LaunchTiming* t = nullptr);
// The sum of the S slabs of src [S][R][Cs] fp32, slabs added in order:
// columns 0 .. C1 - 1 to dst1 [R][C1], C1 .. C1 + C2 - 1 to dst2 [R][C2]
// (storage dtype).
hipError_t launch_sum_slices(int et, const float* src, void* dst1, void* dst2, int S, int R, int Cs, int C1, int C2,
                             hipStream_t s, const LaunchTiming* t = nullptr);
// Zero `bytes` bytes at p (16-byte aligned) with a kernel (no memset node in
// captured graphs).
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s, const LaunchTiming* t = nullptr);
// zr[bh][k] = z[bh][(N - k) mod N] for BH lines of N fp32 values.
hipError_t launch_reverse_lines(const float* z, float* zr, int BH, int N, hipStream_t s,
                                const LaunchTiming* t = nullptr);
// 1D mixing for N beyond one workgroup's line, on a transform of length
// L = L1 L2 (three passes over HBM; see cat_longconv.hip): L = N for a
// power-of-two N, else a power of two >= 2N - 1.
struct LongArgs {
  const float2* tw;  // W_L^m, m < L
  int logL1, logL2;  // L1 = 2^logL1 (column DFTs), L2 = 2^logL2 (row DFTs)
  int BH, pairs;     // (batch, head) lines and channel pairs per head (d / 2)
  int N;             // tokens per line (N == L, or 2N - 1 <= L)
  int H, D, d;
  int pb;            // channel pairs per block of V and of the intermediates (1, 2, 4 or 8; divides pairs)
};
// Launches, in order: softmax chunk partials, column pass and row pass of
// the filter spectrum (zc: partials scratch, at least [BH][ceil(N / 1024)] complex;
// Az: [BH][L] complex fp32 scratch; S: [BH][L] spectrum), then
// column pass, row pass with the spectrum product, inverse column pass of
// the values (V BLOCKED with 2 pb-channel groups, A: [BH d/2][L] complex
// fp32 scratch, O [B][N][D]).  t: six timing slots or null.
hipError_t launch_longconv(int et, const LongArgs& a, const float* logits, const void* V, float2* zc, float2* Az,
                           float2* S, float2* A, void* O, hipStream_t s, const LaunchTiming* const* t = nullptr);
// The score gradient of the long path (mixing backward): with dOb and Vb in
// the blocked layout of the values (2 pb-channel groups),
//   dz*[bh][k] = sum over the head's channels c and tokens i of
//                dO_c[i] V_c[(i - k) mod N]
// as the real part of IDFT_L(sum over pairs of DFT(dO pair) conj DFT(V pair))
// / L (folded onto mod N on a padded circle), then
//   dlogits = z* (dz* - <z*, dz*>),  z* = softmax(logits).
// Ad, Av: [BH d/2][L] complex fp32 scratch; R: [BH][L] complex fp32
// scratch; c: [BH][L] fp32 scratch; dlogits [BH][N] fp32.  t: one timing
// slot for every launch, or null.
hipError_t launch_long_scoregrad(int et, const LongArgs& a, const float* logits, const void* dOb, const void* Vb,
                                 float2* Ad, float2* Av, float2* R, float* c, float* dlogits, hipStream_t s,
                                 const LaunchTiming* t = nullptr);
// 2D: out[bh][k] = sum over g of part[bh][g][k] (partials [BH][ngrp][L],
// out [BH][L], complex fp32; summed in order g = 0, 1, ..).
hipError_t launch_psum(const float2* part, float2* out, int BH, int ngrp, int L, hipStream_t s,
                       const LaunchTiming* t = nullptr);
hipError_t launch_relayout(const RelayoutArgs& a, hipStream_t s, const LaunchTiming* t = nullptr);
// 2D BCCB mixing on the matrix cores (cat_bconv.hip): square grids of side
// G = 32 or 96, bf16 storage, d % 8 == 0.  V BLOCKED with 2-channel groups;
// spec in the transposed order [BH][kr][kc] (kc contiguous), 1/N included;
// table of the plan's bf16 DFT fragments (bconv_table_halfs(G) entries); O
// [B][N][D].
struct BconvArgs {
  const void* V;
  const float2* spec;
  const void* table;
  void* O;
  int BH, npair, H, D, d;
  int num_cu;
  int nfull, nhalf;  // quads, then half-quads (set by launch_bconv)
};
bool bconv_supported(int G);
size_t bconv_table_halfs(int G);
hipError_t launch_bconv(const BconvArgs& a, int G, hipStream_t s, const LaunchTiming* t = nullptr);

// Logits of the averaged-key variant (cat_variants.hip):
//   z[b][h][n] = X[b][n] . (W_Q[:, head h] kbar[b]_h) * scale,
//   kbar[b] = (token mean of X[b]) W_K.
// X [B][N][D], W_Q, W_K [D][D] in the storage dtype; part: at least
// avgkey_part_floats(B, N, D) floats of scratch; kbar [B][D], weff [B][D][H]
// and z [B][H][N] fp32.  D % 8 == 0, D <= 3072, H <= 32, B <= 65535.  t:
// four timing slots or null.
struct AvgKeyArgs {
  const void* X;
  const void* W_Q;
  const void* W_K;
  float* part;
  float* kbar;
  float* weff;
  float* z;
  int B, N, D, H;
  float scale;
};
size_t avgkey_part_floats(int B, int N, int D);
hipError_t launch_avgkey(int et, const AvgKeyArgs& a, hipStream_t s, const LaunchTiming* const* t = nullptr);

// Plan-level helpers of the C-ABI layer (cat_api.cpp) for entry points in
// other translation units.
size_t plan_forward_ws_bytes(const cat_plan_s* plan);
int64_t plan_batch(const cat_plan_s* plan);
cat_status plan_check_forward_1d(const cat_plan_s* plan, const void* X, const void* W_A, const void* W_V,
                                 const void* O);
cat_status forward_1d_checked(cat_plan_s* plan, const void* X, const void* W_A, const void* W_V, void* O,
                              void* workspace, void* stream);
cat_status set_error(cat_status s, const char* msg);

// Raise the dynamic-LDS limit of the kernels a geometry uses (once per plan).
hipError_t prepare_kernels(const LineGeom& g, size_t conv_lds, size_t spec_lds, size_t score_lds);

}  // namespace cat
