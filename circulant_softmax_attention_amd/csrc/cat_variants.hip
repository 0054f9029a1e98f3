// cat_variants.hip -- the logits of the averaged-key variant of CAT.
//
// The CAT page's ablation table compares parameterisations of the circulant
// scores; its "qkv (Averaged-Key)" row keeps all three projections (3 D^2
// parameters) at O(N log N) cost (CAT: Circular-Convolutional Attention for
// Sub-Quadratic Transformers, ablation table).  Read as the key averaged over
// the tokens and met by each query as in scaled dot-product attention:
//
//   Q = X W_Q,  K = X W_K,  kbar_h = (1/N) sum_n K_h[n],
//   z_h[n] = Q_h[n] . kbar_h / sqrt(d),
//
// after which the softmax over n and the circulant mixing of V = X W_V are
// CAT's own.  Because the mean and the products are linear, the same logits
// come without forming Q or K:
//
//   xbar = (1/N) sum_n X[n]            (token mean of the input)
//   kbar = xbar W_K                    (the mean key, D values)
//   w_h  = W_Q[:, head h] kbar_h / sqrt(d)   (D values per head)
//   z_h[n] = X[n] . w_h
//
// so the two D x D projections of every token (4 T D^2 flops) shrink to two
// matrix-vector products per sequence and a rank-H product per token; the
// sums are the definition's, in another association (equal up to fp32
// rounding order).  Five small launches, all fp32 arithmetic:
//   colsum_part_kernel   column sums of X over chunks of 16 tokens
//   xbar_kernel          xbar (chunks summed in order, / N)
//   avgkey_kbar_kernel   kbar = xbar W_K, the K range in four quarters
//   avgkey_weff_kernel   w[b][k][h], one d-long dot product per thread
//   avgkey_logits_kernel z[b][h][n] on fp32 matrix cores, 16 tokens per
//                        wave, heads in blocks of 16
#include "cat_common.hpp"
#include "cat_internal.hpp"

namespace cat {

namespace {

constexpr int TCH = 16;   // tokens per column-sum chunk
constexpr int HMAX = 32;  // heads the logits kernel holds in registers

template <int ET>
__device__ __forceinline__ void load8(const void* base, size_t idx, float (&v)[8]) {
  if constexpr (ET == ET_F32) {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx + 4);
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
    v[0] = bf16lo(u.x), v[1] = bf16hi(u.x), v[2] = bf16lo(u.y), v[3] = bf16hi(u.y);
    v[4] = bf16lo(u.z), v[5] = bf16hi(u.z), v[6] = bf16lo(u.w), v[7] = bf16hi(u.w);
  }
}

template <int ET>
__device__ __forceinline__ float ld1(const void* p, size_t i) {
  if constexpr (ET == ET_F32)
    return reinterpret_cast<const float*>(p)[i];
  else
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
}

// part[b][chunk][k] = sum over the chunk's tokens n of X[b][n][k]; grid
// (chunks, B, column blocks of 2048), each thread 8 adjacent columns, the
// chunk's loads issued together.
template <int ET>
__global__ __launch_bounds__(256) void colsum_part_kernel(const void* __restrict__ X, float* __restrict__ part, int N,
                                                          int D, int nchunk) {
  const int chunk = blockIdx.x, b = blockIdx.y;
  const int k0 = (blockIdx.z * 256 + threadIdx.x) * 8;
  if (k0 >= D) return;
  const int n0 = chunk * TCH, cnt = min(TCH, N - n0);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (cnt == TCH) {
    float v[TCH][8];
#pragma unroll
    for (int i = 0; i < TCH; ++i) load8<ET>(X, ((size_t)b * N + n0 + i) * D + k0, v[i]);
#pragma unroll
    for (int i = 0; i < TCH; ++i)
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += v[i][u];
  } else {
    for (int i = 0; i < cnt; ++i) {
      float v[8];
      load8<ET>(X, ((size_t)b * N + n0 + i) * D + k0, v);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += v[u];
    }
  }
  float* dst = part + ((size_t)b * nchunk + chunk) * D + k0;
  *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// xbar[b][k] = (sum over chunks of part[b][chunk][k]) / N; grid (column
// blocks of 64, B): thread (k, g) sums the g-th quarter of the chunks in
// order (loads issued eight at a time), the quarters are added in order.
__global__ __launch_bounds__(256) void xbar_kernel(const float* __restrict__ part, float* __restrict__ xbar, int N,
                                                   int D, int nchunk) {
  __shared__ float red[4][64];
  const int b = blockIdx.y, lane = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int k = blockIdx.x * 64 + lane;
  const int cq = (nchunk + 3) / 4, c0 = g * cq, c1 = min(nchunk, c0 + cq);
  float s = 0.f;
  if (k < D) {
    const float* src = part + (size_t)b * nchunk * D + k;
    int ch = c0;
    for (; ch + 8 <= c1; ch += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = src[(size_t)(ch + u) * D];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; ch < c1; ++ch) s += src[(size_t)ch * D];
  }
  red[g][lane] = s;
  __syncthreads();
  if (g == 0 && k < D)
    xbar[(size_t)b * D + k] = (((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane]) * (1.f / (float)N);
}

// kbar[b][c] = sum_k xbar[b][k] W_K[k][c]; grid (column blocks of 64, B):
// thread (c, q) sums the q-th quarter of the K range, the quarters are
// added in order.  xbar[b] is staged in LDS (D <= 3072).
template <int ET>
__global__ __launch_bounds__(256) void avgkey_kbar_kernel(const float* __restrict__ xbar, const void* __restrict__ W_K,
                                                          float* __restrict__ kbar, int D) {
  __shared__ float xs[3072];
  __shared__ float red[4][64];
  const int b = blockIdx.y, lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  for (int k = threadIdx.x; k < D; k += 256) xs[k] = xbar[(size_t)b * D + k];
  __syncthreads();
  const int kq = (D + 3) / 4, k0 = q * kq, k1 = min(D, k0 + kq);
  float acc = 0.f;
  if (c < D) {
    int k = k0;
    for (; k + 8 <= k1; k += 8) {  // 8 loads in flight, then their products in order
      float w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = ld1<ET>(W_K, (size_t)(k + u) * D + c);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += xs[k + u] * w[u];
    }
    for (; k < k1; ++k) acc += xs[k] * ld1<ET>(W_K, (size_t)k * D + c);
  }
  red[q][lane] = acc;
  __syncthreads();
  if (q == 0 && c < D) kbar[(size_t)b * D + c] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

// weff[b][k][h] = scale * sum_{j < d} W_Q[k][h d + j] kbar[b][h d + j]; grid
// (blocks of 256 (k, h) pairs, B), one pair per thread; kbar[b] in LDS.
template <int ET>
__global__ __launch_bounds__(256) void avgkey_weff_kernel(const float* __restrict__ kbar, const void* __restrict__ W_Q,
                                                          float* __restrict__ weff, int D, int H, float scale) {
  __shared__ float kb[3072];
  const int b = blockIdx.y;
  for (int c = threadIdx.x; c < D; c += 256) kb[c] = kbar[(size_t)b * D + c];
  __syncthreads();
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= D * H) return;
  const int k = t / H, h = t - k * H, d = D / H;
  const int c0 = h * d;
  float s = 0.f;
  if (d % 32 == 0) {
    for (int j = 0; j < d; j += 32) {  // four 8-value loads in flight
      float w[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i) load8<ET>(W_Q, (size_t)k * D + c0 + j + 8 * i, w[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int u = 0; u < 8; ++u) s += w[i][u] * kb[c0 + j + 8 * i + u];
    }
  } else if (d % 8 == 0) {
    for (int j = 0; j < d; j += 8) {
      float w[8];
      load8<ET>(W_Q, (size_t)k * D + c0 + j, w);
#pragma unroll
      for (int u = 0; u < 8; ++u) s += w[u] * kb[c0 + j + u];
    }
  } else {
    for (int j = 0; j < d; ++j) s += ld1<ET>(W_Q, (size_t)k * D + c0 + j) * kb[c0 + j];
  }
  weff[((size_t)b * D + k) * H + h] = s * scale;
}

// z[b][h][n] = sum_k X[b][n][k] weff[b][k][h] on v_mfma_f32_16x16x4_f32
// (fp32 products, fp32 accumulation); grid (token blocks of 64, B), four
// waves of 16 tokens, heads in blocks of 16 (one or two).  The weff slice of
// KC rows is staged in LDS with 32 heads per row (zero past H; pitch 34).  Lane (i, g)
// of a wave (i = lane % 16, g = lane / 16) supplies, for MFMA m of a K step
// of 32, the A value weff[k][16 hb + i] and the B value X[token i][k] at
// k = 8 g + m: both operands walk the same K positions, so the order inside
// the step does not matter.  The result of lane (i, g), register v, is head
// 16 hb + 4 g + v of token i.
template <int ET>
__global__ __launch_bounds__(256) void avgkey_logits_kernel(const void* __restrict__ X, const float* __restrict__ weff,
                                                            float* __restrict__ z, int N, int D, int H) {
  constexpr int KC = 256;
  constexpr int WP = HMAX + 2;  // row pitch: the four lane groups' rows (8 apart) fall in disjoint banks
  __shared__ float wk[KC * WP];
  typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
  const int b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  const int tok = blockIdx.x * 64 + wave * 16 + li;
  const int tokc = tok < N ? tok : N - 1;  // rows past N load a valid row; their results are not stored
  const int nhb = (H + 15) / 16;
  floatx4 acc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
  const size_t xrow = ((size_t)b * N + tokc) * D;
  // staging: thread t holds head t % 32 of rows t / 32 + 8 j, j < KC / 8
  const int sh = threadIdx.x & (HMAX - 1), sr = threadIdx.x >> 5;
  for (int k0 = 0; k0 < D; k0 += KC) {
    const int kn = min(KC, D - k0);
    // this slice's X runs (8 values per K step of 32), loaded before any is used
    float x[KC / 32][8];
#pragma unroll
    for (int st = 0; st < KC / 32; ++st) {
      const int r0 = 32 * st + 8 * lg;
      load8<ET>(X, xrow + k0 + (r0 < kn ? r0 : 0), x[st]);
    }
    float wv[KC / 8];
#pragma unroll
    for (int j = 0; j < KC / 8; ++j) {
      const int r = sr + 8 * j;
      wv[j] = sh < H && r < kn ? weff[((size_t)b * D + k0 + r) * H + sh] : 0.f;
    }
    __syncthreads();  // the previous slice is consumed
#pragma unroll
    for (int j = 0; j < KC / 8; ++j) wk[(sr + 8 * j) * WP + sh] = wv[j];
    __syncthreads();
#pragma unroll
    for (int st = 0; st < KC / 32; ++st) {
      const int r0 = 32 * st + 8 * lg;  // this lane group's 8 K positions (kn is a multiple of 8)
      const bool ok = r0 < kn;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float bv = ok ? x[st][m] : 0.f;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          if (hb < nhb) {
            const float av = ok ? wk[(r0 + m) * WP + 16 * hb + li] : 0.f;
            acc[hb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[hb], 0, 0, 0);
          }
      }
    }
  }
  if (tok < N)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int h = 16 * hb + 4 * lg + v;
        if (hb < nhb && h < H) z[((size_t)b * H + h) * N + tok] = acc[hb][v];
      }
}

template <int ET>
hipError_t launch_avgkey_et(const AvgKeyArgs& a, hipStream_t s, const LaunchTiming* const* t) {
  const int nchunk = (a.N + TCH - 1) / TCH;
  float* xbar = a.part + (size_t)a.B * nchunk * a.D;
  hipError_t e = launch_k(colsum_part_kernel<ET>, dim3(nchunk, a.B, (a.D + 2047) / 2048), dim3(256), 0, s,
                          t ? t[0] : nullptr, a.X, a.part, a.N, a.D, nchunk);
  if (e != hipSuccess) return e;
  e = launch_k(xbar_kernel, dim3((a.D + 63) / 64, a.B), dim3(256), 0, s, t ? t[1] : nullptr, (const float*)a.part,
               xbar, a.N, a.D, nchunk);
  if (e != hipSuccess) return e;
  e = launch_k(avgkey_kbar_kernel<ET>, dim3((a.D + 63) / 64, a.B), dim3(256), 0, s, t ? t[2] : nullptr,
               (const float*)xbar, a.W_K, a.kbar, a.D);
  if (e != hipSuccess) return e;
  e = launch_k(avgkey_weff_kernel<ET>, dim3((a.D * a.H + 255) / 256, a.B), dim3(256), 0, s, t ? t[3] : nullptr,
               (const float*)a.kbar, a.W_Q, a.weff, a.D, a.H, a.scale);
  if (e != hipSuccess) return e;
  return launch_k(avgkey_logits_kernel<ET>, dim3((a.N + 63) / 64, a.B), dim3(256), 0, s, t ? t[4] : nullptr, a.X,
                  (const float*)a.weff, a.z, a.N, a.D, a.H);
}

}  // namespace

// column-sum partials [B][ceil(N / TCH)][D], then xbar [B][D]
size_t avgkey_part_floats(int B, int N, int D) { return (size_t)B * ((N + TCH - 1) / TCH) * D + (size_t)B * D; }

hipError_t launch_avgkey(int et, const AvgKeyArgs& a, hipStream_t s, const LaunchTiming* const* t) {
  if (a.B < 1 || a.N < 1 || a.D < 8 || a.D % 8 != 0 || a.H < 1 || a.H > HMAX || a.D % a.H != 0 || a.D > 3072)
    return hipErrorInvalidValue;
  if ((long)a.B > 65535 || (long)(a.N + 63) / 64 > 0x7fffffffL || (long)a.D * a.H > 0x7fffffffL)
    return hipErrorInvalidValue;
  return et == ET_F32 ? launch_avgkey_et<ET_F32>(a, s, t) : launch_avgkey_et<ET_BF16>(a, s, t);
}

}  // namespace cat
