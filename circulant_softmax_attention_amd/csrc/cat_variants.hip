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
// rounding order).  Four small launches, all fp32 arithmetic:
//   colsum_part_kernel   column sums of X over chunks of 64 tokens
//   avgkey_kbar_kernel   xbar (chunks summed in order, / N), then kbar
//   avgkey_weff_kernel   w[b][k][h]
//   avgkey_logits_kernel z[b][h][n]
#include "cat_common.hpp"
#include "cat_internal.hpp"

namespace cat {

namespace {

constexpr int TCH = 64;  // tokens per column-sum chunk

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
// (chunks, B, column blocks of 2048), each thread 8 adjacent columns.
template <int ET>
__global__ __launch_bounds__(256) void colsum_part_kernel(const void* __restrict__ X, float* __restrict__ part, int N,
                                                          int D, int nchunk) {
  const int chunk = blockIdx.x, b = blockIdx.y;
  const int k0 = (blockIdx.z * 256 + threadIdx.x) * 8;
  if (k0 >= D) return;
  const int n0 = chunk * TCH, n1 = min(N, n0 + TCH);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int n = n0; n < n1; ++n) {
    float v[8];
    load8<ET>(X, ((size_t)b * N + n) * D + k0, v);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += v[u];
  }
  float* dst = part + ((size_t)b * nchunk + chunk) * D + k0;
  *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// kbar[b][c] = sum_k xbar[b][k] W_K[k][c], xbar[b][k] = (sum over chunks in
// order of part[b][chunk][k]) / N; grid (column blocks of 256, B).  xbar is
// rebuilt in LDS by every workgroup, 1024 entries at a time.
template <int ET>
__global__ __launch_bounds__(256) void avgkey_kbar_kernel(const float* __restrict__ part, const void* __restrict__ W_K,
                                                          float* __restrict__ kbar, int N, int D, int nchunk) {
  __shared__ float xs[1024];
  const int b = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  const float invN = 1.f / (float)N;
  float acc = 0.f;
  for (int k0 = 0; k0 < D; k0 += 1024) {
    const int kn = min(1024, D - k0);
    __syncthreads();  // the previous slice is consumed
    for (int k = threadIdx.x; k < kn; k += 256) {
      float s = 0.f;
      for (int ch = 0; ch < nchunk; ++ch) s += part[((size_t)b * nchunk + ch) * D + k0 + k];
      xs[k] = s * invN;
    }
    __syncthreads();
    if (c < D)
      for (int k = 0; k < kn; ++k) acc += xs[k] * ld1<ET>(W_K, (size_t)(k0 + k) * D + c);
  }
  if (c < D) kbar[(size_t)b * D + c] = acc;
}

// weff[b][k][h] = scale * sum_{c in head h} W_Q[k][c] kbar[b][c]; grid (row
// blocks of 16, B), 4 waves of 4 rows each.  A wave forms the row's D
// products with coalesced reads of W_Q, then lanes h < H add their head's d
// products in order.  Dynamic LDS: kbar (D floats) + 4 product rows.
template <int ET>
__global__ __launch_bounds__(256) void avgkey_weff_kernel(const float* __restrict__ kbar, const void* __restrict__ W_Q,
                                                          float* __restrict__ weff, int D, int H, float scale) {
  extern __shared__ float sm[];
  float* kb = sm;
  const int b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* prod = sm + D + wave * D;
  const int d = D / H;
  for (int c = threadIdx.x; c < D; c += 256) kb[c] = kbar[(size_t)b * D + c];
  __syncthreads();
  for (int r = 0; r < 4; ++r) {
    const int k = blockIdx.x * 16 + wave * 4 + r;  // uniform per wave
    if (k < D)
      for (int c = lane; c < D; c += 64) prod[c] = ld1<ET>(W_Q, (size_t)k * D + c) * kb[c];
    __syncthreads();
    if (k < D && lane < H) {
      float s = 0.f;
      for (int c = 0; c < d; ++c) s += prod[lane * d + c];
      weff[((size_t)b * D + k) * H + lane] = s * scale;
    }
    __syncthreads();  // prod is reused by the next row
  }
}

// z[b][h][n] = sum_k X[b][n][k] weff[b][k][h]; grid (token blocks of 64, B),
// thread (token tid / 4, heads tid % 4 + 4 u).  weff is staged in LDS in
// slices of 256 rows (H <= 32 columns).
template <int ET>
__global__ __launch_bounds__(256) void avgkey_logits_kernel(const void* __restrict__ X, const float* __restrict__ weff,
                                                            float* __restrict__ z, int N, int D, int H) {
  constexpr int KC = 256, HMAX = 32, UMAX = HMAX / 4;
  __shared__ float wk[KC * HMAX];
  const int b = blockIdx.y;
  const int n = blockIdx.x * 64 + (threadIdx.x >> 2), hq = threadIdx.x & 3;
  float acc[UMAX];
#pragma unroll
  for (int u = 0; u < UMAX; ++u) acc[u] = 0.f;
  for (int k0 = 0; k0 < D; k0 += KC) {
    const int kn = min(KC, D - k0);
    __syncthreads();
    for (int i = threadIdx.x; i < kn * H; i += 256) wk[i] = weff[((size_t)b * D + k0) * H + i];
    __syncthreads();
    if (n < N) {
      for (int k = 0; k < kn; k += 8) {  // D % 8 == 0, so slices hold whole runs of 8
        float v[8];
        load8<ET>(X, ((size_t)b * N + n) * D + k0 + k, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float* row = wk + (k + e) * H;
#pragma unroll
          for (int u = 0; u < UMAX; ++u)
            if (hq + 4 * u < H) acc[u] += v[e] * row[hq + 4 * u];
        }
      }
    }
  }
  if (n < N)
#pragma unroll
    for (int u = 0; u < UMAX; ++u)
      if (hq + 4 * u < H) z[((size_t)b * H + hq + 4 * u) * N + n] = acc[u];
}

template <int ET>
hipError_t launch_avgkey_et(const AvgKeyArgs& a, hipStream_t s, const LaunchTiming* const* t) {
  const int nchunk = (a.N + TCH - 1) / TCH;
  hipError_t e = launch_k(colsum_part_kernel<ET>, dim3(nchunk, a.B, (a.D + 2047) / 2048), dim3(256), 0, s,
                          t ? t[0] : nullptr, a.X, a.part, a.N, a.D, nchunk);
  if (e != hipSuccess) return e;
  e = launch_k(avgkey_kbar_kernel<ET>, dim3((a.D + 255) / 256, a.B), dim3(256), 0, s, t ? t[1] : nullptr, a.part,
               a.W_K, a.kbar, a.N, a.D, nchunk);
  if (e != hipSuccess) return e;
  e = launch_k(avgkey_weff_kernel<ET>, dim3((a.D + 15) / 16, a.B), dim3(256), (size_t)5 * a.D * sizeof(float), s,
               t ? t[2] : nullptr, a.kbar, a.W_Q, a.weff, a.D, a.H, a.scale);
  if (e != hipSuccess) return e;
  return launch_k(avgkey_logits_kernel<ET>, dim3((a.N + 63) / 64, a.B), dim3(256), 0, s, t ? t[3] : nullptr, a.X,
                  a.weff, a.z, a.N, a.D, a.H);
}

}  // namespace

size_t avgkey_part_floats(int B, int N, int D) { return (size_t)B * ((N + TCH - 1) / TCH) * D; }

hipError_t launch_avgkey(int et, const AvgKeyArgs& a, hipStream_t s, const LaunchTiming* const* t) {
  if (a.B < 1 || a.N < 1 || a.D < 8 || a.D % 8 != 0 || a.H < 1 || a.H > 32 || a.D % a.H != 0 || a.D > 3072)
    return hipErrorInvalidValue;
  if ((long)a.B > 65535 || (long)(a.N + 63) / 64 > 0x7fffffffL) return hipErrorInvalidValue;
  return et == ET_F32 ? launch_avgkey_et<ET_F32>(a, s, t) : launch_avgkey_et<ET_BF16>(a, s, t);
}

}  // namespace cat
