// cat_longconv.hip -- the 1D circulant mixing for sequences longer than one
// workgroup's transform line (power-of-two N with 4096 < N <= 65536, other
// N with 2048 < N <= 32768).
//
// CAT evaluates O_h = circ(z*_h) V_h as IFFT(FFT(z*_h) . FFT(V_h)) along the
// tokens (CAT: Circular-Convolutional Attention for Sub-Quadratic
// Transformers, "Key designs: FFT-accelerated computation"); the page names
// sequences beyond 10^4 tokens as where that O(N log N) route should pay.
// A length L = L1 L2 transform does not fit one workgroup here, so it runs
// as three passes over HBM (four-step FFT), with L = N for a power-of-two
// N.  Any other N runs exactly on a power-of-two circle L >= 2N - 1: the
// values are zero-padded to L, the softmax line is wrapped (entry j < N at
// j, entry N - m at L - m for 0 < m < N, zeros between), and the first N
// outputs of the length-L circular product are the length-N ones:
//
//   column pass   for each n2: A[k1][n2] = W_L^(k1 n2) sum_n1 x[n1 L2 + n2] W_L1^(n1 k1)
//   row pass      for each k1: X[k1 + L1 k2] = sum_n2 A[k1][n2] W_L2^(n2 k2);
//                 times S[k1 + L1 k2] (the filter spectrum over L), then the
//                 inverse over k2 back to B[k1][n2]
//   inverse column pass  for each n2: o[n1 L2 + n2] = sum_k1 B[k1][n2] conj W_L^(k1 n2) conj W_L1^(n1 k1)
//
// The filter spectrum is the column pass and the forward half of the row
// pass applied to the softmax line, scaled by 1/L; the softmax is reduced
// in chunks first, and the column pass normalises the logits as it loads
// them.  A short DFT of square length (64 or 256) runs as a register
// four-step: sqrt(M) lanes per line, a register DFT over each lane's
// values, the twiddle, one exchange through LDS and a second register DFT;
// other lengths (128) run as a Stockham transform in LDS (radix-4 stages,
// one radix-2 stage when log2 of the length is odd; natural order in and
// out), several lines per workgroup.  All twiddles come from one table
// W_L^m, m < L, computed in double precision on the host.  Two real
// channels ride in one complex line, as in the single-workgroup
// convolution.
//
// Layouts: V is BLOCKED with 2 PB-channel groups ([BH][d/2/PB][N][PB]
// complex, PB channel pairs per block); O is [B][N][D]; the intermediate A is
// [BH][d/2/PB][L1][L2][PB] complex fp32; the spectrum S is [BH][L1][L2]
// complex fp32 (entry k1 L2 + k2 holds frequency k1 + L1 k2).
#include "cat_common.hpp"
#include "cat_internal.hpp"

namespace cat {

namespace {

constexpr int LTHR = 256;
constexpr int LBUF = 2048;  // complex values of the lines one workgroup transforms
constexpr int LPAD = LBUF + 64;  // LDS buffer size: lines at pitch M + 1 (at most 64 lines)
constexpr int LMAXM = 256;       // longest short DFT (L1, L2 <= 256: N <= 65536)

__device__ __forceinline__ float2 cmul2(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}
__device__ __forceinline__ float2 conj2(float2 a) { return make_float2(a.x, -a.y); }

// Stockham stages of an M-point transform: one radix-2 stage first when
// log2 M is odd, then radix-4 stages with Ns = 1 or 2, then x4 up to M.
// The radix-4 stage twiddles live in LDS: the stage with span Ns holds, at
// offset toff(Ns) + 3 k + r - 1, W_(4 Ns)^(r k) = W_L^(r k L / (4 Ns)) for
// k < Ns, r = 1..3 (at most 255 entries for M <= 256).  Read by lds_fft
// after its first barrier.
__device__ __forceinline__ void stage_twiddles(float2* tws, int logM, const float2* __restrict__ tw, int logL) {
  const int M = 1 << logM, L = 1 << logL;
  int Ns = (logM & 1) ? 2 : 1, toff = 0;
  for (; Ns < M; toff += 3 * Ns, Ns *= 4) {
    const int step = L / (4 * Ns);
    for (int i = threadIdx.x; i < 3 * Ns; i += LTHR) {
      const int k = i / 3, r = i - 3 * k + 1;
      tws[toff + i] = tw[(r * k * step) & (L - 1)];
    }
  }
}

// R independent lines of M points (M a power of two) at a[r (M + 1) + i]
// (the odd pitch keeps column-wise accesses off a single bank), natural
// order in and out, unscaled; b is the ping-pong buffer; tws the stage
// twiddles (stage_twiddles).  Returns the buffer holding the result.  Ends
// with a barrier.
template <bool INV>
__device__ float2* lds_fft(float2* a, float2* b, int M, int logM, int R, const float2* tws) {
  const int P = M + 1;
  int Ns = 1, toff = 0;
  if (logM & 1) {  // radix 2, span 1: no twiddle
    const int half = M >> 1;
    __syncthreads();
    for (int q = threadIdx.x; q < R * half; q += LTHR) {
      const int r = q >> (logM - 1), j = q & (half - 1);
      const float2 v0 = a[r * P + j], v1 = a[r * P + j + half];
      b[r * P + 2 * j] = make_float2(v0.x + v1.x, v0.y + v1.y);
      b[r * P + 2 * j + 1] = make_float2(v0.x - v1.x, v0.y - v1.y);
    }
    float2* t = a;
    a = b;
    b = t;
    Ns = 2;
  }
  const int quarter = M >> 2;
  const int lq = logM - 2;
  for (; Ns < M; toff += 3 * Ns, Ns *= 4) {
    __syncthreads();
    for (int q = threadIdx.x; q < R * quarter; q += LTHR) {
      const int r = q >> lq, j = q & (quarter - 1);
      const int k = j & (Ns - 1);
      const float2* src = a + r * P + j;
      float2 v0 = src[0], v1 = src[quarter], v2 = src[2 * quarter], v3 = src[3 * quarter];
      float2 w1 = tws[toff + 3 * k], w2 = tws[toff + 3 * k + 1], w3 = tws[toff + 3 * k + 2];
      if (INV) {
        w1 = conj2(w1);
        w2 = conj2(w2);
        w3 = conj2(w3);
      }
      v1 = cmul2(v1, w1);
      v2 = cmul2(v2, w2);
      v3 = cmul2(v3, w3);
      const float2 t0 = make_float2(v0.x + v2.x, v0.y + v2.y), t1 = make_float2(v0.x - v2.x, v0.y - v2.y);
      const float2 t2 = make_float2(v1.x + v3.x, v1.y + v3.y), t3 = make_float2(v1.x - v3.x, v1.y - v3.y);
      // forward W_4 = -i: X1 = t1 - i t3, X3 = t1 + i t3 (inverse: swapped)
      const float2 mt3 = INV ? make_float2(-t3.y, t3.x) : make_float2(t3.y, -t3.x);  // -/+ i t3
      float2* dst = b + r * P + ((j & ~(Ns - 1)) << 2) + k;
      dst[0] = make_float2(t0.x + t2.x, t0.y + t2.y);
      dst[Ns] = make_float2(t1.x + mt3.x, t1.y + mt3.y);
      dst[2 * Ns] = make_float2(t0.x - t2.x, t0.y - t2.y);
      dst[3 * Ns] = make_float2(t1.x - mt3.x, t1.y - mt3.y);
    }
    float2* t = a;
    a = b;
    b = t;
  }
  __syncthreads();
  return a;
}

template <int ET>
__device__ __forceinline__ float2 load_c(const void* base, size_t i) {
  if constexpr (ET == ET_F32) {
    return reinterpret_cast<const float2*>(base)[i];
  } else {
    const uint32_t u = reinterpret_cast<const uint32_t*>(base)[i];
    return make_float2(bf16lo(u), bf16hi(u));
  }
}

// Entry j of the softmax line on the transform circle: the line itself when
// L = N; otherwise its wrapped extension (z*[j] for j < N, z*[j - (L - N)]
// for j > L - N, zero between; L >= 2N - 1 keeps the two ranges apart).
// zl: the line's logits; ms: (max, 1 / sum of exp).
// The load is clamped to a valid token and the zero selected afterwards, so
// no load sits behind a branch and all of a thread's loads issue together.
__device__ __forceinline__ float circle_score(const float* __restrict__ zl, int j, int N, int L, float2 ms) {
  const int n = j < N ? j : j > L - N ? j - (L - N) : -1;
  const float v = __expf(zl[n < 0 ? 0 : n] - ms.x) * ms.y;
  return n < 0 ? 0.f : v;
}

// ---- softmax partials: chunk c (SMC logits, the last one ragged) of line
// bh -> (max m_c, sum exp(z - m_c)); the column pass of the spectrum
// combines the chunks of its line and normalises on the fly.
constexpr int SMC = 1024;
__host__ __device__ constexpr int smc_chunks(int N) { return (N + SMC - 1) / SMC; }
__global__ __launch_bounds__(LTHR) void softmax_part_kernel(const float* __restrict__ z, float2* __restrict__ part,
                                                            int N) {
  __shared__ float red[LTHR / 64];
  const int nc = smc_chunks(N);
  const int bh = blockIdx.x / nc, c = blockIdx.x - bh * nc, tid = threadIdx.x;
  const float* zr = z + (size_t)bh * N + (size_t)c * SMC;
  const int len = N - c * SMC;  // >= 1; entries past it are -inf and add nothing
  float v[SMC / LTHR];
#pragma unroll
  for (int i = 0; i < SMC / LTHR; ++i) v[i] = tid + LTHR * i < len ? zr[tid + LTHR * i] : -INFINITY;
  auto reduce = [&](float x, bool is_max) {
    for (int o = 32; o >= 1; o >>= 1) {
      const float p = __shfl_xor(x, o, 64);
      x = is_max ? fmaxf(x, p) : x + p;
    }
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = x;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < LTHR / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
    return r;
  };
  float m = v[0];
#pragma unroll
  for (int i = 1; i < SMC / LTHR; ++i) m = fmaxf(m, v[i]);
  m = reduce(m, true);
  float se = 0.f;
#pragma unroll
  for (int i = 0; i < SMC / LTHR; ++i) se += __expf(v[i] - m);
  se = reduce(se, false);
  if (tid == 0) part[blockIdx.x] = make_float2(m, se);
}

// Pair blocks.  The values' lines come in blocks of PB channel pairs with
// the pair index innermost: V [BH][P / PB][N][PB] (the blocked layout with
// 2 PB-channel groups) and A [BH][P / PB][L1][L2][PB], so that one token (or
// one (k1, n2) point) of a block is PB contiguous complex values.  A
// workgroup transforms every pair of its block; the spectrum's line is a
// block of one.

// ---- column pass: CB adjacent columns n2 of block `gl`, every pair:
// A[gl][k1][n2][j] = W_L^(k1 n2) DFT_L1 over n1 of x[n1 L2 + n2][j].
// SET: ET_F32 (float2 values), ET_BF16 (bf16 pairs), or 2 (fp32 logits,
// softmax from the chunk partials; PB = 1).  WRAP: the line is shorter than
// the circle (values zero past N, the softmax line wrapped); without it
// L = N and every load is a plain one.
template <int SET, bool WRAP>
__global__ __launch_bounds__(LTHR) void col_fwd_kernel(LongArgs a, int PB, const void* __restrict__ src,
                                                       float2* __restrict__ A, const float2* __restrict__ smpart) {
  __shared__ float2 buf[2][LPAD];
  __shared__ float2 tws[LMAXM];
  __shared__ float2 msum;
  const int L1 = 1 << a.logL1, L2 = 1 << a.logL2, L = L1 * L2;
  const int CB = LBUF / (PB * L1) < L2 ? LBUF / (PB * L1) : L2, R = CB * PB;
  const int nblk = L2 / CB;
  const int gl = blockIdx.x / nblk, n20 = (blockIdx.x - gl * nblk) * CB;
  const size_t gbase = (size_t)gl * L * PB;
  if constexpr (SET == 2) {
    // softmax of the line from its chunk partials: m = max m_c,
    // s = sum s_c exp(m_c - m); one wave combines them
    const int nc = smc_chunks(a.N);
    if (threadIdx.x < 64) {
      float2 p = threadIdx.x < nc ? smpart[(size_t)gl * nc + threadIdx.x] : make_float2(-INFINITY, 0.f);
      float m = p.x;
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      float sv = threadIdx.x < nc ? p.y * __expf(p.x - m) : 0.f;
      for (int o = 32; o >= 1; o >>= 1) sv += __shfl_xor(sv, o, 64);
      if (threadIdx.x == 0) msum = make_float2(m, 1.f / sv);
    }
    __syncthreads();
  }
  // line r = c PB + j of the workgroup holds column n20 + c of pair j:
  // buf[0][r (L1 + 1) + n1]; consecutive threads read consecutive memory
  for (int q = threadIdx.x; q < R * L1; q += LTHR) {
    const int n1 = q / R, r = q - n1 * R;
    const int j = n1 * L2 + n20 + r / PB;  // position on the circle
    if constexpr (!WRAP) {  // L = N
      const size_t i = gbase + ((size_t)n1 * L2 + n20) * PB + r;
      if constexpr (SET == 2)
        buf[0][r * (L1 + 1) + n1] = make_float2(__expf(reinterpret_cast<const float*>(src)[i] - msum.x) * msum.y, 0.f);
      else
        buf[0][r * (L1 + 1) + n1] = load_c<SET>(src, i);
    } else if constexpr (SET == 2) {
      buf[0][r * (L1 + 1) + n1] =
          make_float2(circle_score(reinterpret_cast<const float*>(src) + (size_t)gl * a.N, j, a.N, L, msum), 0.f);
    } else {
      // clamped load, then select (past N: zero padding)
      const bool ok = j < a.N;
      const float2 v = load_c<SET>(src, (size_t)gl * a.N * PB + (ok ? ((size_t)n1 * L2 + n20) * PB : 0) + r);
      buf[0][r * (L1 + 1) + n1] = ok ? v : make_float2(0.f, 0.f);
    }
  }
  stage_twiddles(tws, a.logL1, a.tw, a.logL1 + a.logL2);
  const float2* U = lds_fft<false>(buf[0], buf[1], L1, a.logL1, R, tws);
  for (int q = threadIdx.x; q < R * L1; q += LTHR) {
    const int k1 = q / R, r = q - k1 * R;
    const int n2 = n20 + r / PB;
    const float2 w = a.tw[(k1 * n2) & (L - 1)];
    A[gbase + ((size_t)k1 * L2 + n20) * PB + r] = cmul2(U[r * (L1 + 1) + k1], w);
  }
}

// ---- row pass, RB rows k1 of block `gl` per workgroup, every pair.
// MODE 0 (spectrum, PB = 1): S = DFT_L2 / L of the rows of Az.  MODE 1
// (mixing): A = IDFT_L2(DFT_L2(A) . S[bh]) in place, bh = gl / (P / PB).
template <int MODE>
__global__ __launch_bounds__(LTHR) void row_kernel(LongArgs a, int PB, float2* __restrict__ A, float2* __restrict__ S) {
  __shared__ float2 buf[2][LPAD];
  __shared__ float2 tws[LMAXM];
  const int L1 = 1 << a.logL1, L2 = 1 << a.logL2, L = L1 * L2;
  const int RB = LBUF / (PB * L2) < L1 ? LBUF / (PB * L2) : L1, R = RB * PB;
  const int nblk = L1 / RB;
  const int gl = blockIdx.x / nblk, k10 = (blockIdx.x - gl * nblk) * RB;
  const size_t base = ((size_t)gl * L + (size_t)k10 * L2) * PB;  // RB contiguous rows of the block
  const int P2 = L2 + 1;
  // LDS line r = (k1 - k10) PB + j: row k1 of pair j, buf[r P2 + n2]
  const int RL = L2 * PB;  // values per row of the block
  for (int q = threadIdx.x; q < RB * RL; q += LTHR) {
    const int rr = q / RL, rem = q - rr * RL, n2 = rem / PB, j = rem - n2 * PB;
    buf[0][(rr * PB + j) * P2 + n2] = A[base + q];
  }
  stage_twiddles(tws, a.logL2, a.tw, a.logL1 + a.logL2);
  float2* X = lds_fft<false>(buf[0], buf[1], L2, a.logL2, R, tws);
  float2* Y = X == buf[0] ? buf[1] : buf[0];
  if constexpr (MODE == 0) {
    const float sc = 1.f / (float)L;
    for (int q = threadIdx.x; q < RB * L2; q += LTHR) {
      const int rr = q >> a.logL2, k2 = q & (L2 - 1);
      const float2 v = X[rr * P2 + k2];
      S[base + q] = make_float2(v.x * sc, v.y * sc);
    }
  } else {
    const size_t sbase = (size_t)(gl / (a.pairs / PB)) * L + (size_t)k10 * L2;
    for (int q = threadIdx.x; q < R * L2; q += LTHR) {
      const int r = q >> a.logL2, k2 = q & (L2 - 1);
      const int i = r * P2 + k2;
      X[i] = cmul2(X[i], S[sbase + (size_t)(r / PB) * L2 + k2]);
    }
    const float2* Bv = lds_fft<true>(X, Y, L2, a.logL2, R, tws);
    for (int q = threadIdx.x; q < RB * RL; q += LTHR) {
      const int rr = q / RL, rem = q - rr * RL, n2 = rem / PB, j = rem - n2 * PB;
      A[base + q] = Bv[(rr * PB + j) * P2 + n2];
    }
  }
}

// ---- register four-step transform of one line of M = MS^2 points, held
// by MS lanes: lane t holds element ma MS + t in register ma (ma < MS).
// DFT over ma in registers, twiddle W_M^(ka t), exchange through the
// line's [MS][MS + 1] LDS tile, DFT over the other digit: lane t then holds
// X[t + MS kb] in register kb.  That output layout is the input layout of
// the next transform (high digit in the register), so a forward and an
// inverse transform chain with no reordering.  xl: the line's LDS tile;
// twm: W_M^e, e < M.  Ends with a barrier.
template <int MS, bool INV>
__device__ __forceinline__ void reg_fft(cf* x, int t, float2* xl, const float2* twm) {
  constexpr int M = MS * MS;
  Dft<MS, INV>::run(x);
#pragma unroll
  for (int ka = 1; ka < MS; ++ka) {
    const float2 w = twm[(ka * t) & (M - 1)];
    x[ka] = INV ? cmulc(x[ka], cfm(w.x, w.y)) : cmul(x[ka], cfm(w.x, w.y));
  }
#pragma unroll
  for (int ka = 0; ka < MS; ++ka) xl[ka * (MS + 1) + t] = make_float2(x[ka].x, x[ka].y);
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < MS; ++mb) {
    const float2 v = xl[t * (MS + 1) + mb];
    x[mb] = cfm(v.x, v.y);
  }
  __syncthreads();  // the tile may be reused
  Dft<MS, INV>::run(x);
}

// Pitch (complex values) of one line's LDS tile in a workgroup of R lines,
// lane r = tid % R of each line fastest: at least MS (MS + 1), and congruent
// to 32 / R modulo 32 (1 when R >= 32).  The 32 lanes of a half-wave (R
// lines, 32 / R consecutive t) then fall on 32 distinct 8-byte bank pairs,
// both where the tile is written (index r TP + ka (MS + 1) + t) and where
// it is read transposed (index r TP + t (MS + 1) + mb).  With the bare
// MS (MS + 1) the lines' tiles started on one or two bank pairs.
template <int MS, int R>
constexpr int tile_pitch() {
  constexpr int base = MS * (MS + 1), want = R >= 32 ? 1 : 32 / R;
  return base + ((want - base) % 32 + 32) % 32;
}

// The values' intermediate A between the passes: complex fp32 (float2), or,
// for bf16 storage on the all-register path, a bf16 pair (real part in the
// low half) that halves the passes' traffic.  Arithmetic stays fp32.
__device__ __forceinline__ float2 lda(const float2* p, size_t i) { return p[i]; }
__device__ __forceinline__ float2 lda(const uint32_t* p, size_t i) {
  const uint32_t w = p[i];
  return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}
__device__ __forceinline__ void sta(float2* p, size_t i, float2 v) { p[i] = v; }
__device__ __forceinline__ void sta(uint32_t* p, size_t i, float2 v) { p[i] = pack_bf16x2(v.x, v.y); }

// ---- row pass on registers (L2 = MS^2), 128 threads: R = 128 / MS lines
// (rows x pairs) per workgroup, lane r = tid % R of each line fastest so a
// wave's loads and stores are contiguous.  MODE as row_kernel.
template <int MODE, int MS, class AT = float2>
__global__ __launch_bounds__(128) void row_reg_kernel(LongArgs a, int PB, AT* __restrict__ A,
                                                      float2* __restrict__ S) {
  constexpr int M = MS * MS, R = 128 / MS, TP = tile_pitch<MS, R>();
  __shared__ float2 xb[R * TP];
  __shared__ float2 twm[M];
  const int L1 = 1 << a.logL1, L = L1 * M;
  const int RB = R / PB;  // rows per workgroup
  const int nblk = L1 / RB;
  const int gl = blockIdx.x / nblk, k10 = (blockIdx.x - gl * nblk) * RB;
  const size_t base = ((size_t)gl * L + (size_t)k10 * M) * PB;
  const int r = threadIdx.x % R, t = threadIdx.x / R;
  const int rr = r / PB, j = r - rr * PB;
  for (int e = threadIdx.x; e < M; e += 128) twm[e] = a.tw[e * (L / M)];
  cf x[MS];
#pragma unroll
  for (int ma = 0; ma < MS; ++ma) {
    const float2 v = lda(A, base + ((size_t)rr * M + ma * MS + t) * PB + j);
    x[ma] = cfm(v.x, v.y);
  }
  __syncthreads();  // twiddles in LDS
  float2* xl = xb + r * TP;
  reg_fft<MS, false>(x, t, xl, twm);
  if constexpr (MODE == 0) {
    const float sc = 1.f / (float)L;
#pragma unroll
    for (int kb = 0; kb < MS; ++kb)
      S[base + (size_t)rr * M + t + MS * kb] = make_float2(x[kb].x * sc, x[kb].y * sc);
  } else {
    const size_t sbase = (size_t)(gl / (a.pairs / PB)) * L + (size_t)(k10 + rr) * M;
#pragma unroll
    for (int kb = 0; kb < MS; ++kb) x[kb] = cmul(x[kb], *reinterpret_cast<const cf*>(&S[sbase + t + MS * kb]));
    reg_fft<MS, true>(x, t, xl, twm);
#pragma unroll
    for (int nb = 0; nb < MS; ++nb)
      sta(A, base + ((size_t)rr * M + t + MS * nb) * PB + j, make_float2(x[nb].x, x[nb].y));
  }
}

// ---- column passes on registers (L1 = MS^2), 128 threads: R = 128 / MS
// lines (CB = R / PB columns x PB pairs) per workgroup, lane r fastest.
// Forward: SET as col_fwd_kernel.  Lane t of line r = c PB + j holds
// x[(ma MS + t) L2 + n20 + c][j] in register ma; after the transform it
// holds k1 = t + MS kb in register kb.
template <int SET, int MS, bool WRAP, class AT = float2, int NT = 128>
__global__ __launch_bounds__(NT) void col_reg_kernel(LongArgs a, int PB, const void* __restrict__ src,
                                                     AT* __restrict__ A, const float2* __restrict__ smpart) {
  constexpr int M = MS * MS, R = NT / MS, TP = tile_pitch<MS, R>();
  __shared__ float2 xb[R * TP];
  __shared__ float2 twm[M];
  __shared__ float2 msum;
  const int L2 = 1 << a.logL2, L = M * L2;
  const int CB = R / PB;
  const int nblk = L2 / CB;
  const int gl = blockIdx.x / nblk, n20 = (blockIdx.x - gl * nblk) * CB;
  const size_t gbase = (size_t)gl * L * PB;
  const int r = threadIdx.x % R, t = threadIdx.x / R;
  const int c = r / PB;
  for (int e = threadIdx.x; e < M; e += NT) twm[e] = a.tw[e * (L / M)];
  if constexpr (SET == 2) {
    const int nc = smc_chunks(a.N);
    if (threadIdx.x < 64) {
      float2 p = threadIdx.x < nc ? smpart[(size_t)gl * nc + threadIdx.x] : make_float2(-INFINITY, 0.f);
      float m = p.x;
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      float sv = threadIdx.x < nc ? p.y * __expf(p.x - m) : 0.f;
      for (int o = 32; o >= 1; o >>= 1) sv += __shfl_xor(sv, o, 64);
      if (threadIdx.x == 0) msum = make_float2(m, 1.f / sv);
    }
  }
  __syncthreads();  // twiddles (and the softmax constants) in LDS
  cf x[MS];
#pragma unroll
  for (int ma = 0; ma < MS; ++ma) {
    const int n = (ma * MS + t) * L2 + n20;
    float2 v;
    if constexpr (!WRAP) {  // L = N
      const size_t i = gbase + (size_t)n * PB + r;
      if constexpr (SET == 2)
        v = make_float2(__expf(reinterpret_cast<const float*>(src)[i] - msum.x) * msum.y, 0.f);
      else
        v = load_c<SET>(src, i);
    } else if constexpr (SET == 2) {
      v = make_float2(circle_score(reinterpret_cast<const float*>(src) + (size_t)gl * a.N, n + c, a.N, L, msum), 0.f);
    } else {
      // clamped load, then select (past N: zero padding)
      const bool ok = n + c < a.N;
      v = load_c<SET>(src, (size_t)gl * a.N * PB + (ok ? (size_t)n * PB : 0) + r);
      v = ok ? v : make_float2(0.f, 0.f);
    }
    x[ma] = cfm(v.x, v.y);
  }
  reg_fft<MS, false>(x, t, xb + r * TP, twm);
  const int n2 = n20 + c;
#pragma unroll
  for (int kb = 0; kb < MS; ++kb) {
    const int k1 = t + MS * kb;
    const float2 w = a.tw[(k1 * n2) & (L - 1)];
    const cf y = cmul(x[kb], cfm(w.x, w.y));
    sta(A, gbase + ((size_t)k1 * L2 + n20) * PB + r, make_float2(y.x, y.y));
  }
}

// Inverse column pass on registers: lane t of line r holds
// A[k1][n2][j] conj W_L^(k1 n2) for k1 = ma MS + t in register ma; after the
// inverse transform it holds n1 = t + MS nb in register nb, written to O.
template <int DET, int MS, class AT = float2, int NT = 128>
__global__ __launch_bounds__(NT) void col_inv_reg_kernel(LongArgs a, int PB, const AT* __restrict__ A,
                                                         void* __restrict__ O) {
  constexpr int M = MS * MS, R = NT / MS, TP = tile_pitch<MS, R>();
  __shared__ float2 xb[R * TP];
  __shared__ float2 twm[M];
  const int L2 = 1 << a.logL2, L = M * L2;
  const int CB = R / PB;
  const int nblk = L2 / CB;
  const int gl = blockIdx.x / nblk, n20 = (blockIdx.x - gl * nblk) * CB;
  const size_t gbase = (size_t)gl * L * PB;
  const int r = threadIdx.x % R, t = threadIdx.x / R;
  const int c = r / PB, j = r - c * PB;
  const int n2 = n20 + c;
  for (int e = threadIdx.x; e < M; e += NT) twm[e] = a.tw[e * (L / M)];
  cf x[MS];
#pragma unroll
  for (int ma = 0; ma < MS; ++ma) {
    const int k1 = ma * MS + t;
    const float2 v = lda(A, gbase + ((size_t)k1 * L2 + n20) * PB + r);
    const float2 w = a.tw[(k1 * n2) & (L - 1)];
    x[ma] = cmulc(cfm(v.x, v.y), cfm(w.x, w.y));
  }
  __syncthreads();  // twiddles in LDS
  reg_fft<MS, true>(x, t, xb + r * TP, twm);
  const int groups = a.pairs / PB;
  const int bh = gl / groups, g = gl - bh * groups;
  const int b = bh / a.H, h = bh - b * a.H;
  const size_t obase = (size_t)b * a.N * a.D + (size_t)h * a.d + 2 * ((size_t)g * PB + j);
#pragma unroll
  for (int nb = 0; nb < MS; ++nb) {
    const int n = (t + MS * nb) * L2 + n2;
    if (n >= a.N) continue;  // past the line: the padded circle's tail
    if constexpr (DET == ET_F32) {
      *reinterpret_cast<float2*>(reinterpret_cast<float*>(O) + obase + n * a.D) = make_float2(x[nb].x, x[nb].y);
    } else {
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(O) + obase + n * a.D) = pack_bf16x2(x[nb].x, x[nb].y);
    }
  }
}

// ---- inverse column pass: o[n1 L2 + n2][j] = IDFT_L1 over k1 of
// A[gl][k1][n2][j] conj W_L^(k1 n2), written to O[b][n][h d + 2 (g PB + j) ..]
// (storage element type DET), gl = bh (P / PB) + g.
template <int DET>
__global__ __launch_bounds__(LTHR) void col_inv_kernel(LongArgs a, int PB, const float2* __restrict__ A,
                                                       void* __restrict__ O) {
  __shared__ float2 buf[2][LPAD];
  __shared__ float2 tws[LMAXM];
  const int L1 = 1 << a.logL1, L2 = 1 << a.logL2, L = L1 * L2;
  const int CB = LBUF / (PB * L1) < L2 ? LBUF / (PB * L1) : L2, R = CB * PB;
  const int nblk = L2 / CB;
  const int gl = blockIdx.x / nblk, n20 = (blockIdx.x - gl * nblk) * CB;
  const size_t gbase = (size_t)gl * L * PB;
  for (int q = threadIdx.x; q < R * L1; q += LTHR) {
    const int k1 = q / R, r = q - k1 * R;
    const int n2 = n20 + r / PB;
    buf[0][r * (L1 + 1) + k1] =
        cmul2(A[gbase + ((size_t)k1 * L2 + n20) * PB + r], conj2(a.tw[(k1 * n2) & (L - 1)]));
  }
  stage_twiddles(tws, a.logL1, a.tw, a.logL1 + a.logL2);
  const float2* U = lds_fft<true>(buf[0], buf[1], L1, a.logL1, R, tws);
  const int groups = a.pairs / PB;
  const int bh = gl / groups, g = gl - bh * groups;
  const int b = bh / a.H, h = bh - b * a.H;
  const size_t obase = (size_t)b * a.N * a.D + (size_t)h * a.d + 2 * (size_t)g * PB;
  for (int q = threadIdx.x; q < R * L1; q += LTHR) {
    const int n1 = q / R, r = q - n1 * R;
    const int c = r / PB, j = r - c * PB;
    const int n = n1 * L2 + n20 + c;
    if (n >= a.N) continue;  // past the line: the padded circle's tail
    const float2 v = U[r * (L1 + 1) + n1];
    if constexpr (DET == ET_F32) {
      *reinterpret_cast<float2*>(reinterpret_cast<float*>(O) + obase + n * a.D + 2 * j) = v;
    } else {
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(O) + obase + n * a.D + 2 * j) = pack_bf16x2(v.x, v.y);
    }
  }
}


// ---- score gradient (mixing backward).  The circular cross-correlation
// of two complex lines p, q is IDFT(DFT(p) conj DFT(q)) / L:
//   r[m] = sum_i p[i] conj(q[i - m]),
// and with p = a + i b, q = c + i d (two real channels each) its real part
// is sum_i a[i] c[i - m] + b[i] d[i - m], the correlation summed over both
// channels of the pair.  Summing the products over every pair of a head
// before one inverse transform gives the head's dz* line.
//
// Row pass: RB rows k1 of head bh per workgroup, all pair blocks in turn:
// the forward DFT over n2 of the rows of Ad (kept) and of Av, the products
// Ad conj(Av) summed over the pairs into acc, and at the end the inverse DFT
// over k2 of the RB summed rows:  R[bh][k1][n2].
__global__ __launch_bounds__(LTHR) void row_xcorr_kernel(LongArgs a, int PB, const float2* __restrict__ Ad,
                                                         const float2* __restrict__ Av, float2* __restrict__ R) {
  __shared__ float2 buf[2][LPAD];
  __shared__ float2 keep[LPAD];
  __shared__ float2 acc[LBUF];
  __shared__ float2 tws[LMAXM];
  const int L1 = 1 << a.logL1, L2 = 1 << a.logL2, L = L1 * L2;
  const int RB = LBUF / (PB * L2) < L1 ? LBUF / (PB * L2) : L1, Rn = RB * PB;
  const int nblk = L1 / RB;
  const int bh = blockIdx.x / nblk, k10 = (blockIdx.x - bh * nblk) * RB;
  const int groups = a.pairs / PB;
  const int P2 = L2 + 1, RL = L2 * PB;
  for (int q = threadIdx.x; q < RB * L2; q += LTHR) acc[q] = make_float2(0.f, 0.f);
  stage_twiddles(tws, a.logL2, a.tw, a.logL1 + a.logL2);
  for (int g = 0; g < groups; ++g) {
    const size_t base = (((size_t)bh * groups + g) * L + (size_t)k10 * L2) * PB;  // RB contiguous rows
    for (int q = threadIdx.x; q < RB * RL; q += LTHR) {
      const int rr = q / RL, rem = q - rr * RL, n2 = rem / PB, j = rem - n2 * PB;
      buf[0][(rr * PB + j) * P2 + n2] = Ad[base + q];
    }
    const float2* X = lds_fft<false>(buf[0], buf[1], L2, a.logL2, Rn, tws);
    for (int q = threadIdx.x; q < Rn * L2; q += LTHR) {
      const int r = q >> a.logL2, k2 = q & (L2 - 1);
      keep[r * P2 + k2] = X[r * P2 + k2];
    }
    __syncthreads();  // X (possibly buf[0]) is consumed before buf[0] is refilled
    for (int q = threadIdx.x; q < RB * RL; q += LTHR) {
      const int rr = q / RL, rem = q - rr * RL, n2 = rem / PB, j = rem - n2 * PB;
      buf[0][(rr * PB + j) * P2 + n2] = Av[base + q];
    }
    const float2* Y = lds_fft<false>(buf[0], buf[1], L2, a.logL2, Rn, tws);
    for (int q = threadIdx.x; q < RB * L2; q += LTHR) {
      const int rr = q >> a.logL2, k2 = q & (L2 - 1);
      float2 sum = acc[q];
      for (int j = 0; j < PB; ++j) {
        const int i = (rr * PB + j) * P2 + k2;
        sum.x += keep[i].x * Y[i].x + keep[i].y * Y[i].y;
        sum.y += keep[i].y * Y[i].x - keep[i].x * Y[i].y;
      }
      acc[q] = sum;
    }
    __syncthreads();  // keep and the buffers are reused by the next block
  }
  for (int q = threadIdx.x; q < RB * L2; q += LTHR) {
    const int rr = q >> a.logL2, k2 = q & (L2 - 1);
    buf[0][rr * P2 + k2] = acc[q];
  }
  const float2* Bv = lds_fft<true>(buf[0], buf[1], L2, a.logL2, RB, tws);
  const size_t obase = (size_t)bh * L + (size_t)k10 * L2;
  for (int q = threadIdx.x; q < RB * L2; q += LTHR) {
    const int rr = q >> a.logL2, n2 = q & (L2 - 1);
    R[obase + q] = Bv[rr * P2 + n2];
  }
}

// Inverse column pass of the summed line: c[bh][n1 L2 + n2] = Re(IDFT_L1
// over k1 of R[bh][k1][n2] conj W_L^(k1 n2)) / L, CB columns per workgroup.
__global__ __launch_bounds__(LTHR) void col_inv_corr_kernel(LongArgs a, const float2* __restrict__ R,
                                                            float* __restrict__ c) {
  __shared__ float2 buf[2][LPAD];
  __shared__ float2 tws[LMAXM];
  const int L1 = 1 << a.logL1, L2 = 1 << a.logL2, L = L1 * L2;
  const int CB = LBUF / L1 < L2 ? LBUF / L1 : L2;
  const int nblk = L2 / CB;
  const int bh = blockIdx.x / nblk, n20 = (blockIdx.x - bh * nblk) * CB;
  const size_t gbase = (size_t)bh * L;
  for (int q = threadIdx.x; q < CB * L1; q += LTHR) {
    const int k1 = q / CB, r = q - k1 * CB;
    const int n2 = n20 + r;
    buf[0][r * (L1 + 1) + k1] = cmul2(R[gbase + (size_t)k1 * L2 + n2], conj2(a.tw[(k1 * n2) & (L - 1)]));
  }
  stage_twiddles(tws, a.logL1, a.tw, a.logL1 + a.logL2);
  const float2* U = lds_fft<true>(buf[0], buf[1], L1, a.logL1, CB, tws);
  const float sc = 1.f / (float)L;
  for (int q = threadIdx.x; q < CB * L1; q += LTHR) {
    const int n1 = q / CB, r = q - n1 * CB;
    c[gbase + (size_t)n1 * L2 + n20 + r] = U[r * (L1 + 1) + n1].x * sc;
  }
}

// dlogits[bh][k] = z*[k] (g[k] - sum_m z*[m] g[m]) with z* = softmax of the
// line's logits and g[k] = c[k] (+ c[L - N + k] for 0 < k < N on a padded
// circle: lags that wrap mod N land there).  One 1024-thread workgroup per
// line; four passes over the line (max, sum, dot, write).
constexpr int GTHR = 1024;
__device__ __forceinline__ float block_reduce(float x, bool is_max, float* red) {
  for (int o = 32; o >= 1; o >>= 1) {
    const float p = __shfl_xor(x, o, 64);
    x = is_max ? fmaxf(x, p) : x + p;
  }
  __syncthreads();  // red is free
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < GTHR / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}
__global__ __launch_bounds__(GTHR) void logits_grad_long_kernel(const float* __restrict__ z, const float* __restrict__ c,
                                                                float* __restrict__ dz, int N, int L) {
  __shared__ float red[GTHR / 64];
  const int bh = blockIdx.x;
  const float* zl = z + (size_t)bh * N;
  const float* cl = c + (size_t)bh * L;
  const bool wrap = N != L;
  float m = -INFINITY;
  for (int k = threadIdx.x; k < N; k += GTHR) m = fmaxf(m, zl[k]);
  m = block_reduce(m, true, red);
  float se = 0.f;
  for (int k = threadIdx.x; k < N; k += GTHR) se += __expf(zl[k] - m);
  const float inv = 1.f / block_reduce(se, false, red);
  auto grad = [&](int k) { return cl[k] + (wrap && k > 0 ? cl[L - N + k] : 0.f); };
  float dot = 0.f;
  for (int k = threadIdx.x; k < N; k += GTHR) dot += __expf(zl[k] - m) * inv * grad(k);
  dot = block_reduce(dot, false, red);
  for (int k = threadIdx.x; k < N; k += GTHR) {
    const float p = __expf(zl[k] - m) * inv;
    dz[(size_t)bh * N + k] = p * (grad(k) - dot);
  }
}

// The value column pass (forward): src BLOCKED values -> A, PB pairs per
// block; register kernels when L1 is 64 or 256.
hipError_t launch_col_values(int et, const LongArgs& a, const void* src, float2* A, hipStream_t s,
                             const LaunchTiming* t) {
  const int L1 = 1 << a.logL1, L2 = 1 << a.logL2, L = L1 * L2, PB = a.pb;
  const bool wrap = a.N != L;
  const long blocks = (long)a.BH * (a.pairs / PB);
  const float2* nosm = nullptr;
  const int mc = L1 == 256 ? 16 : L1 == 64 ? 8 : 0;
  auto col = [&](auto plain, auto wrapped, unsigned grid, unsigned threads) {
    return wrap ? launch_k(wrapped, dim3(grid), dim3(threads), 0, s, t, a, PB, src, A, nosm)
                : launch_k(plain, dim3(grid), dim3(threads), 0, s, t, a, PB, src, A, nosm);
  };
  if (mc) {
    const unsigned cv = (unsigned)(blocks * (L2 / ((128 / mc) / PB)));
    if (mc == 16)
      return et == ET_F32 ? col(col_reg_kernel<ET_F32, 16, false>, col_reg_kernel<ET_F32, 16, true>, cv, 128)
                          : col(col_reg_kernel<ET_BF16, 16, false>, col_reg_kernel<ET_BF16, 16, true>, cv, 128);
    return et == ET_F32 ? col(col_reg_kernel<ET_F32, 8, false>, col_reg_kernel<ET_F32, 8, true>, cv, 128)
                        : col(col_reg_kernel<ET_BF16, 8, false>, col_reg_kernel<ET_BF16, 8, true>, cv, 128);
  }
  const int cb = LBUF / (PB * L1) < L2 ? LBUF / (PB * L1) : L2;
  const unsigned colb = (unsigned)(blocks * (L2 / cb));
  return et == ET_F32 ? col(col_fwd_kernel<ET_F32, false>, col_fwd_kernel<ET_F32, true>, colb, LTHR)
                      : col(col_fwd_kernel<ET_BF16, false>, col_fwd_kernel<ET_BF16, true>, colb, LTHR);
}

// Shape checks shared by the long launchers.
bool long_shape_ok(const LongArgs& a) {
  const int L1 = 1 << a.logL1, L2 = 1 << a.logL2, L = L1 * L2, N = a.N, PB = a.pb;
  if (a.logL1 < 1 || a.logL2 < 1 || L1 > LMAXM || L2 > LMAXM || a.pairs < 1 || a.BH < 1) return false;
  if (PB < 1 || PB > 8 || (PB & (PB - 1)) != 0 || a.pairs % PB != 0) return false;
  const int cb1 = LBUF / L1 < L2 ? LBUF / L1 : L2, rb1 = LBUF / L2 < L1 ? LBUF / L2 : L1;
  const int cb = LBUF / (PB * L1) < L2 ? LBUF / (PB * L1) : L2, rb = LBUF / (PB * L2) < L1 ? LBUF / (PB * L2) : L1;
  if (cb < 1 || rb < 1 || cb1 > 64 || rb1 > 64 || cb * PB > 64 || rb * PB > 64) return false;
  if (N < 1 || (N != L && 2 * N - 1 > L) || smc_chunks(N) > 64) return false;
  const long blocks = (long)a.BH * (a.pairs / PB);
  return blocks * (L2 / cb) <= 0x7fffffffL && blocks * (L1 / rb) <= 0x7fffffffL;
}

}  // namespace

hipError_t launch_longconv(int et, const LongArgs& a, const float* logits, const void* V, float2* zc, float2* Az,
                           float2* S, float2* A, void* O, hipStream_t s, const LaunchTiming* const* t) {
  const LaunchTiming* none[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  if (!t) t = none;
  const int L1 = 1 << a.logL1, L2 = 1 << a.logL2, L = L1 * L2, N = a.N, PB = a.pb;
  if (a.logL1 < 1 || a.logL2 < 1 || L1 > LMAXM || L2 > LMAXM || a.pairs < 1 || a.BH < 1) return hipErrorInvalidValue;
  if (PB < 1 || PB > 8 || (PB & (PB - 1)) != 0 || a.pairs % PB != 0) return hipErrorInvalidValue;
  // lines per workgroup (CB PB columns, RB PB rows) stay within the LDS pad
  const int cb1 = LBUF / L1 < L2 ? LBUF / L1 : L2, rb1 = LBUF / L2 < L1 ? LBUF / L2 : L1;
  const int cb = LBUF / (PB * L1) < L2 ? LBUF / (PB * L1) : L2, rb = LBUF / (PB * L2) < L1 ? LBUF / (PB * L2) : L1;
  if (cb < 1 || rb < 1 || cb1 > 64 || rb1 > 64 || cb * PB > 64 || rb * PB > 64) return hipErrorInvalidValue;
  // the line fills the circle, or fits on it twice less one (the wrapped product)
  if (N < 1 || (N != L && 2 * N - 1 > L) || smc_chunks(N) > 64) return hipErrorInvalidValue;
  const long blocks = (long)a.BH * (a.pairs / PB);
  const long colb_z = (long)a.BH * (L2 / cb1), rowb_z = (long)a.BH * (L1 / rb1);
  const long colb = blocks * (L2 / cb), rowb = blocks * (L1 / rb);
  if (colb > 0x7fffffffL || rowb > 0x7fffffffL) return hipErrorInvalidValue;
  // the filter spectrum: softmax partials (in zc), then the column pass of
  // the normalised line, straight from the logits, then the rows
  hipError_t e = launch_k(softmax_part_kernel, dim3((unsigned)(a.BH * smc_chunks(N))), dim3(LTHR), 0, s, t[0], logits, zc, N);
  if (e != hipSuccess) return e;
  // column passes on registers when L1 is a square of 8 or 16 (C = 128 / sqrt(L1) lines per workgroup)
  const bool wrap = N != L;
  auto col = [&](auto plain, auto wrapped, unsigned grid, unsigned threads, const LaunchTiming* tt, int pb,
                 const void* src, auto* dst, const float2* sm) {
    return wrap ? launch_k(wrapped, dim3(grid), dim3(threads), 0, s, tt, a, pb, src, dst, sm)
                : launch_k(plain, dim3(grid), dim3(threads), 0, s, tt, a, pb, src, dst, sm);
  };
  const int mc = L1 == 256 ? 16 : L1 == 64 ? 8 : 0;
  const int cl = mc ? 128 / mc : 0;
  if (mc) {
    const unsigned cz = (unsigned)((long)a.BH * (L2 / cl));
    if (mc == 16)
      e = col(col_reg_kernel<2, 16, false>, col_reg_kernel<2, 16, true>, cz, 128, t[1], 1, (const void*)logits, Az,
              (const float2*)zc);
    else
      e = col(col_reg_kernel<2, 8, false>, col_reg_kernel<2, 8, true>, cz, 128, t[1], 1, (const void*)logits, Az,
              (const float2*)zc);
  } else {
    e = col(col_fwd_kernel<2, false>, col_fwd_kernel<2, true>, (unsigned)colb_z, LTHR, t[1], 1, (const void*)logits, Az,
            (const float2*)zc);
  }
  if (e != hipSuccess) return e;
  // row passes on registers when L2 is a square of 8 or 16 (R = 128 / sqrt(L2) lines per workgroup)
  const int ms = L2 == 256 ? 16 : L2 == 64 ? 8 : 0;
  const int rl = ms ? 128 / ms : 0;
  if (ms) {
    const long rz = (long)a.BH * (L1 / rl);
    if (ms == 16)
      e = launch_k(row_reg_kernel<0, 16>, dim3((unsigned)rz), dim3(128), 0, s, t[2], a, 1, Az, S);
    else
      e = launch_k(row_reg_kernel<0, 8>, dim3((unsigned)rz), dim3(128), 0, s, t[2], a, 1, Az, S);
  } else {
    e = launch_k(row_kernel<0>, dim3((unsigned)rowb_z), dim3(LTHR), 0, s, t[2], a, 1, Az, S);
  }
  if (e != hipSuccess) return e;
  // the mixing, PB pairs per block
  const unsigned cv = mc ? (unsigned)(blocks * (L2 / (cl / PB))) : 0;
  const float2* nosm = nullptr;
  if (et == ET_BF16 && mc && ms) {
    // bf16 storage with both passes on registers: bf16-pair intermediates,
    // and 256-thread column workgroups (2 x 128 / sqrt(L1) lines, so that a
    // point's lines form runs of at least 64 bytes in V and A when PB = 8)
    uint32_t* Ah = reinterpret_cast<uint32_t*>(A);
    const long rv = blocks * (L1 / (rl / PB));
    const unsigned cv2 = (unsigned)(blocks * (L2 / ((256 / mc) / PB)));
    if (mc == 16)
      e = col(col_reg_kernel<ET_BF16, 16, false, uint32_t, 256>, col_reg_kernel<ET_BF16, 16, true, uint32_t, 256>, cv2, 256,
              t[3], PB, V, Ah, nosm);
    else
      e = col(col_reg_kernel<ET_BF16, 8, false, uint32_t, 256>, col_reg_kernel<ET_BF16, 8, true, uint32_t, 256>, cv2, 256,
              t[3], PB, V, Ah, nosm);
    if (e != hipSuccess) return e;
    if (ms == 16)
      e = launch_k(row_reg_kernel<1, 16, uint32_t>, dim3((unsigned)rv), dim3(128), 0, s, t[4], a, PB, Ah, S);
    else
      e = launch_k(row_reg_kernel<1, 8, uint32_t>, dim3((unsigned)rv), dim3(128), 0, s, t[4], a, PB, Ah, S);
    if (e != hipSuccess) return e;
    if (mc == 16)
      return launch_k(col_inv_reg_kernel<ET_BF16, 16, uint32_t, 256>, dim3(cv2), dim3(256), 0, s, t[5], a, PB,
                      (const uint32_t*)Ah, O);
    return launch_k(col_inv_reg_kernel<ET_BF16, 8, uint32_t, 256>, dim3(cv2), dim3(256), 0, s, t[5], a, PB,
                    (const uint32_t*)Ah, O);
  }
  if (mc == 16)
    e = et == ET_F32 ? col(col_reg_kernel<ET_F32, 16, false>, col_reg_kernel<ET_F32, 16, true>, cv, 128, t[3], PB, V, A, nosm)
                     : col(col_reg_kernel<ET_BF16, 16, false>, col_reg_kernel<ET_BF16, 16, true>, cv, 128, t[3], PB, V, A,
                           nosm);
  else if (mc == 8)
    e = et == ET_F32 ? col(col_reg_kernel<ET_F32, 8, false>, col_reg_kernel<ET_F32, 8, true>, cv, 128, t[3], PB, V, A, nosm)
                     : col(col_reg_kernel<ET_BF16, 8, false>, col_reg_kernel<ET_BF16, 8, true>, cv, 128, t[3], PB, V, A,
                           nosm);
  else if (et == ET_F32)
    e = col(col_fwd_kernel<ET_F32, false>, col_fwd_kernel<ET_F32, true>, (unsigned)colb, LTHR, t[3], PB, V, A, nosm);
  else
    e = col(col_fwd_kernel<ET_BF16, false>, col_fwd_kernel<ET_BF16, true>, (unsigned)colb, LTHR, t[3], PB, V, A, nosm);
  if (e != hipSuccess) return e;
  if (ms) {
    const long rv = blocks * (L1 / (rl / PB));
    if (ms == 16)
      e = launch_k(row_reg_kernel<1, 16>, dim3((unsigned)rv), dim3(128), 0, s, t[4], a, PB, A, S);
    else
      e = launch_k(row_reg_kernel<1, 8>, dim3((unsigned)rv), dim3(128), 0, s, t[4], a, PB, A, S);
  } else {
    e = launch_k(row_kernel<1>, dim3((unsigned)rowb), dim3(LTHR), 0, s, t[4], a, PB, A, S);
  }
  if (e != hipSuccess) return e;
  if (mc == 16)
    return et == ET_F32 ? launch_k(col_inv_reg_kernel<ET_F32, 16>, dim3((unsigned)cv), dim3(128), 0, s, t[5], a, PB,
                                   (const float2*)A, O)
                        : launch_k(col_inv_reg_kernel<ET_BF16, 16>, dim3((unsigned)cv), dim3(128), 0, s, t[5], a, PB,
                                   (const float2*)A, O);
  if (mc == 8)
    return et == ET_F32 ? launch_k(col_inv_reg_kernel<ET_F32, 8>, dim3((unsigned)cv), dim3(128), 0, s, t[5], a, PB,
                                   (const float2*)A, O)
                        : launch_k(col_inv_reg_kernel<ET_BF16, 8>, dim3((unsigned)cv), dim3(128), 0, s, t[5], a, PB,
                                   (const float2*)A, O);
  if (et == ET_F32)
    return launch_k(col_inv_kernel<ET_F32>, dim3((unsigned)colb), dim3(LTHR), 0, s, t[5], a, PB, (const float2*)A, O);
  return launch_k(col_inv_kernel<ET_BF16>, dim3((unsigned)colb), dim3(LTHR), 0, s, t[5], a, PB, (const float2*)A, O);
}

hipError_t launch_long_scoregrad(int et, const LongArgs& a, const float* logits, const void* dOb, const void* Vb,
                                 float2* Ad, float2* Av, float2* R, float* c, float* dlogits, hipStream_t s,
                                 const LaunchTiming* t) {
  if (!long_shape_ok(a)) return hipErrorInvalidValue;
  const int L1 = 1 << a.logL1, L2 = 1 << a.logL2, L = L1 * L2;
  hipError_t e = launch_col_values(et, a, dOb, Ad, s, t);
  if (e != hipSuccess) return e;
  if ((e = launch_col_values(et, a, Vb, Av, s, t)) != hipSuccess) return e;
  const int rb = LBUF / (a.pb * L2) < L1 ? LBUF / (a.pb * L2) : L1;
  const int cb1 = LBUF / L1 < L2 ? LBUF / L1 : L2;
  if ((e = launch_k(row_xcorr_kernel, dim3((unsigned)((long)a.BH * (L1 / rb))), dim3(LTHR), 0, s, t, a, a.pb,
                    (const float2*)Ad, (const float2*)Av, R)) != hipSuccess)
    return e;
  if ((e = launch_k(col_inv_corr_kernel, dim3((unsigned)((long)a.BH * (L2 / cb1))), dim3(LTHR), 0, s, t, a,
                    (const float2*)R, c)) != hipSuccess)
    return e;
  return launch_k(logits_grad_long_kernel, dim3((unsigned)a.BH), dim3(GTHR), 0, s, t, logits, (const float*)c, dlogits,
                  a.N, L);
}

}  // namespace cat
