// cat_backward.hip -- layout kernels of the CAT backward's projection
// gradients.  With V = X W_V and z_h = X W_A[:, h] (CAT:
// Circular-Convolutional Attention for Sub-Quadratic Transformers, "Method
// details / Overall framework"), the chain rule gives
//   dX = dV W_V^T + dz^T W_A^T,  dW_V = X^T dV,  dW_A = X^T dz^T,
// i.e. with P = [dV | dz^T] two products on the projection GEMM:
//   [dW_V | dW_A] = X^T P  (K = B N, split into slices summed afterwards),
//   dX = P [W_V^T ; W_A^T]  (K = D + H);
// these kernels build the operands (transposes, P) and sum the slices.
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

// P [B N][D + Hp] (storage dtype) = [dV | dz token-major | 0]: one thread
// per 16-byte chunk of P (D and Hp are multiples of 8, so a chunk lies
// wholly in the dV part or wholly in the dz part).
template <int ET>
__global__ __launch_bounds__(256) void pack_grads_kernel(const void* __restrict__ dV, const float* __restrict__ dz,
                                                         void* __restrict__ P, int B, int N, int D, int H, int Hp) {
  constexpr int VE = ET == ET_F32 ? 4 : 8;
  const int W = D + Hp, cpr = W / VE;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t M = (size_t)B * N;
  if (idx >= M * cpr) return;
  const size_t m = idx / cpr;
  const int c0 = (int)(idx - m * cpr) * VE;
  uint4 v;
  if (c0 < D) {
    v = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(dV) + (m * D + c0) * (ET == ET_F32 ? 4 : 2));
  } else {
    const int b = (int)(m / N), n = (int)(m - (size_t)b * N);
    float f[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const int h = c0 - D + e;
      f[e] = h < H ? dz[((size_t)b * H + h) * N + n] : 0.f;
    }
    if constexpr (ET == ET_F32)
      v = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
    else
      v = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
  }
  reinterpret_cast<uint4*>(P)[idx] = v;
}

unsigned blocks_for(size_t n) { return (unsigned)((n + 255) / 256); }

// The split-K partial products summed: over s = 0, 1, .. S - 1 in order,
// src [S][R][Cs] fp32; columns 0 .. C1 - 1 go to dst1 [R][C1] and columns
// C1 .. C1 + C2 - 1 to dst2 [R][C2] (storage dtype).
template <int ET>
__global__ __launch_bounds__(256) void sum_slices_kernel(const float* __restrict__ src, void* __restrict__ dst1,
                                                         void* __restrict__ dst2, int S, int R, int Cs, int C1, int C2) {
  const int C = C1 + C2;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)R * C) return;
  const size_t r = idx / C;
  const int c = (int)(idx - r * C);
  const size_t slab = (size_t)R * Cs;
  float acc = 0.f;
  for (int k = 0; k < S; ++k) acc += src[k * slab + r * Cs + c];
  if (c < C1)
    st_elem<ET>(dst1, r * C1 + c, acc);
  else
    st_elem<ET>(dst2, r * C2 + (c - C1), acc);
}

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
  const size_t n = (size_t)B * N * ((D + Hp) / (et == ET_F32 ? 4 : 8));  // 16-byte chunks
  if (n == 0 || Hp < H || D % 8 != 0 || Hp % 8 != 0 || blocks_for(n) > 0x7fffffffu) return hipErrorInvalidValue;
  return et == ET_F32
             ? launch_k(pack_grads_kernel<ET_F32>, dim3(blocks_for(n)), dim3(256), 0, s, t, dV, dz, P, B, N, D, H, Hp)
             : launch_k(pack_grads_kernel<ET_BF16>, dim3(blocks_for(n)), dim3(256), 0, s, t, dV, dz, P, B, N, D, H, Hp);
}

hipError_t launch_sum_slices(int et, const float* src, void* dst1, void* dst2, int S, int R, int Cs, int C1, int C2,
                             hipStream_t s, const LaunchTiming* t) {
  const size_t n = (size_t)R * (C1 + C2);
  if (n == 0 || S < 1 || C1 + C2 > Cs || blocks_for(n) > 0x7fffffffu) return hipErrorInvalidValue;
  return et == ET_F32 ? launch_k(sum_slices_kernel<ET_F32>, dim3(blocks_for(n)), dim3(256), 0, s, t, src, dst1, dst2, S,
                                 R, Cs, C1, C2)
                      : launch_k(sum_slices_kernel<ET_BF16>, dim3(blocks_for(n)), dim3(256), 0, s, t, src, dst1, dst2,
                                 S, R, Cs, C1, C2);
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s, const LaunchTiming* t) {
  if (bytes == 0) return hipSuccess;
  const size_t nb = blocks_for((bytes + 15) / 16);
  if (nb > 0x7fffffffu) return hipErrorInvalidValue;
  return launch_k(zero_kernel, dim3((unsigned)nb), dim3(256), 0, s, t, reinterpret_cast<unsigned char*>(p), bytes);
}

}  // namespace cat
