// cat_backward.hip -- layout and elementwise kernels of the CAT backward's
// projection gradients.  With V = X W_V and z_h = X W_A[:, h] (CAT:
// Circular-Convolutional Attention for Sub-Quadratic Transformers, "Method
// details / Overall framework"), the chain rule gives
//   dX = dV W_V^T + dz^T W_A^T,  dW_V = X^T dV,  dW_A = X^T dz^T;
// the products run on the projection GEMM (dW_V and dW_A as two output
// segments of one launch sharing the row operand X^T), and these kernels
// supply its operands and the rank-H term.
#include "cat_common.hpp"
#include "cat_internal.hpp"

namespace cat {

namespace {

template <int ET>
__device__ __forceinline__ float ld_elem(const void* p, size_t i) {
  if constexpr (ET == ET_F32)
    return reinterpret_cast<const float*>(p)[i];
  else
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
}

template <int ET>
__device__ __forceinline__ void st_elem(void* p, size_t i, float v) {
  if constexpr (ET == ET_F32)
    reinterpret_cast<float*>(p)[i] = v;
  else
    reinterpret_cast<uint16_t*>(p)[i] = to_bf16(v);
}

// dst [C][ldd] = src [R][C]^T, storage dtype, with dst columns R .. ldd - 1
// zero; 32 x 32 tiles through LDS (one workgroup per tile, 1D grid of tiles
// over ldd x C).
template <int ET>
__global__ __launch_bounds__(256) void transpose_kernel(const void* __restrict__ src, void* __restrict__ dst, int R,
                                                        int C, int ldd) {
  __shared__ float tile[32][33];
  const int tcs = (C + 31) / 32;
  const int tr = blockIdx.x / tcs, tc = blockIdx.x - tr * tcs;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int k = ty; k < 32; k += 8) {
    const int r = tr * 32 + k, c = tc * 32 + tx;
    if (c < C) tile[k][tx] = r < R ? ld_elem<ET>(src, (size_t)r * C + c) : 0.f;
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int c = tc * 32 + k, r = tr * 32 + tx;
    if (r < ldd && c < C) st_elem<ET>(dst, (size_t)c * ldd + r, tile[tx][k]);
  }
}

// P [B N][D + Hp] (storage dtype) = [dV | dz token-major | 0]: the column
// operand of the product X^T P = [dW_V | dW_A | 0].
template <int ET>
__global__ __launch_bounds__(256) void pack_grads_kernel(const void* __restrict__ dV, const float* __restrict__ dz,
                                                         void* __restrict__ P, int B, int N, int D, int H, int Hp) {
  const int W = D + Hp;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)B * N * W) return;
  const size_t m = idx / W;
  const int col = (int)(idx - m * W);
  float v;
  if (col < D) {
    v = ld_elem<ET>(dV, m * D + col);
  } else {
    const int h = col - D;
    const int b = (int)(m / N), n = (int)(m - (size_t)b * N);
    v = h < H ? dz[((size_t)b * H + h) * N + n] : 0.f;
  }
  st_elem<ET>(P, idx, v);
}

// dX[m][c] = dXf[m][c] + sum_h dz[b][h][n] W_A[c][h]  (m = b N + n, H <= 32),
// in the storage dtype.  A workgroup takes RB token rows: their dz values
// go to LDS (zero past H), each thread keeps its column's W_A row in
// registers and walks the rows, so dXf and dX move in coalesced rows.
constexpr int RB = 16;
template <int ET>
__global__ __launch_bounds__(256) void rank_heads_add_kernel(const float* __restrict__ dXf, const float* __restrict__ dz,
                                                             const void* __restrict__ W_A, void* __restrict__ dX,
                                                             int B, int N, int D, int H) {
  __shared__ float dzs[RB][33];
  const int M = B * N, m0 = blockIdx.x * RB;
  const int rows = M - m0 < RB ? M - m0 : RB;
  for (int i = threadIdx.x; i < RB * 32; i += 256) {
    const int r = i >> 5, h = i & 31;
    float v = 0.f;
    if (r < rows && h < H) {
      const int m = m0 + r, b = m / N, n = m - b * N;
      v = dz[((size_t)b * H + h) * N + n];
    }
    dzs[r][h] = v;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += 256) {
    float w[32];
#pragma unroll
    for (int h = 0; h < 32; ++h) w[h] = h < H ? ld_elem<ET>(W_A, (size_t)c * H + h) : 0.f;
    for (int r = 0; r < rows; ++r) {
      const size_t i = (size_t)(m0 + r) * D + c;
      float acc = dXf[i];
#pragma unroll
      for (int h = 0; h < 32; ++h) acc = fmaf(dzs[r][h], w[h], acc);
      st_elem<ET>(dX, i, acc);
    }
  }
}

// dst [R][Cd] = the first Cd columns of src [R][Cs], storage dtype.
template <int ET>
__global__ __launch_bounds__(256) void take_cols_kernel(const void* __restrict__ src, void* __restrict__ dst, int R,
                                                        int Cs, int Cd) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)R * Cd) return;
  const size_t r = idx / Cd;
  const int c = (int)(idx - r * Cd);
  st_elem<ET>(dst, idx, ld_elem<ET>(src, r * Cs + c));
}

unsigned blocks_for(size_t n) { return (unsigned)((n + 255) / 256); }

// Zero n bytes at p (16-byte aligned): 16-byte stores, then the byte tail.
__global__ __launch_bounds__(256) void zero_kernel(unsigned char* __restrict__ p, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (16 * i + 16 <= n) {
    reinterpret_cast<uint4*>(p)[i] = make_uint4(0u, 0u, 0u, 0u);
  } else {
    for (size_t b = 16 * i; b < n; ++b) p[b] = 0;
  }
}

}  // namespace

hipError_t launch_transpose(int et, const void* src, void* dst, int R, int C, int ldd, hipStream_t s,
                            const LaunchTiming* t) {
  if (R < 1 || C < 1 || ldd < R) return hipErrorInvalidValue;
  const size_t tiles = (size_t)((ldd + 31) / 32) * ((C + 31) / 32);
  if (tiles > 0x7fffffffu) return hipErrorInvalidValue;
  return et == ET_F32 ? launch_k(transpose_kernel<ET_F32>, dim3((unsigned)tiles), dim3(256), 0, s, t, src, dst, R, C, ldd)
                      : launch_k(transpose_kernel<ET_BF16>, dim3((unsigned)tiles), dim3(256), 0, s, t, src, dst, R, C,
                                 ldd);
}

hipError_t launch_pack_grads(int et, const void* dV, const float* dz, void* P, int B, int N, int D, int H, int Hp,
                             hipStream_t s, const LaunchTiming* t) {
  const size_t n = (size_t)B * N * (D + Hp);
  if (n == 0 || Hp < H || blocks_for(n) > 0x7fffffffu) return hipErrorInvalidValue;
  return et == ET_F32
             ? launch_k(pack_grads_kernel<ET_F32>, dim3(blocks_for(n)), dim3(256), 0, s, t, dV, dz, P, B, N, D, H, Hp)
             : launch_k(pack_grads_kernel<ET_BF16>, dim3(blocks_for(n)), dim3(256), 0, s, t, dV, dz, P, B, N, D, H, Hp);
}

hipError_t launch_rank_heads_add(int et, const float* dXf, const float* dz, const void* W_A, void* dX, int B, int N,
                                 int D, int H, hipStream_t s, const LaunchTiming* t) {
  const size_t nb = ((size_t)B * N + RB - 1) / RB;
  if (nb == 0 || H > 32 || nb > 0x7fffffffu) return hipErrorInvalidValue;
  return et == ET_F32
             ? launch_k(rank_heads_add_kernel<ET_F32>, dim3((unsigned)nb), dim3(256), 0, s, t, dXf, dz, W_A, dX, B, N, D, H)
             : launch_k(rank_heads_add_kernel<ET_BF16>, dim3((unsigned)nb), dim3(256), 0, s, t, dXf, dz, W_A, dX, B, N, D,
                        H);
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s, const LaunchTiming* t) {
  if (bytes == 0) return hipSuccess;
  const size_t nb = blocks_for((bytes + 15) / 16);
  if (nb > 0x7fffffffu) return hipErrorInvalidValue;
  return launch_k(zero_kernel, dim3((unsigned)nb), dim3(256), 0, s, t, reinterpret_cast<unsigned char*>(p), bytes);
}

hipError_t launch_take_cols(int et, const void* src, void* dst, int R, int Cs, int Cd, hipStream_t s,
                            const LaunchTiming* t) {
  const size_t n = (size_t)R * Cd;
  if (n == 0 || Cd > Cs || blocks_for(n) > 0x7fffffffu) return hipErrorInvalidValue;
  return et == ET_F32 ? launch_k(take_cols_kernel<ET_F32>, dim3(blocks_for(n)), dim3(256), 0, s, t, src, dst, R, Cs, Cd)
                      : launch_k(take_cols_kernel<ET_BF16>, dim3(blocks_for(n)), dim3(256), 0, s, t, src, dst, R, Cs, Cd);
}

}  // namespace cat
