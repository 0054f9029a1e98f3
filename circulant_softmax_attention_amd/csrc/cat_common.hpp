// cat_common.hpp -- small device helpers shared by the kernel translation units.
#pragma once

#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "cat_fft.hpp"

namespace cat {

// bf16 <-> fp32.  bf16 is the upper half of an fp32 bit pattern; the
// narrowing conversion rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __hip_bfloat162 p = __float22bfloat162_rn(make_float2(a, b));
  return *reinterpret_cast<uint32_t*>(&p);
}
__device__ __forceinline__ uint16_t to_bf16(float a) {
  __hip_bfloat16 p = __float2bfloat16(a);
  return *reinterpret_cast<uint16_t*>(&p);
}

// Complex pair (channels c, c+1 of one token) as one complex value.
template <int ET>
__device__ __forceinline__ cf load_pair(const void* base, size_t idx);
template <>
__device__ __forceinline__ cf load_pair<0>(const void* base, size_t idx) {
  const float2 v = reinterpret_cast<const float2*>(base)[idx / 2];
  return cfm(v.x, v.y);
}
template <>
__device__ __forceinline__ cf load_pair<1>(const void* base, size_t idx) {
  const uint32_t u = reinterpret_cast<const uint32_t*>(base)[idx / 2];
  return cfm(bf16lo(u), bf16hi(u));
}
template <int ET>
__device__ __forceinline__ void store_pair(void* base, size_t idx, cf v);
template <>
__device__ __forceinline__ void store_pair<0>(void* base, size_t idx, cf v) {
  reinterpret_cast<float2*>(base)[idx / 2] = make_float2(v.x, v.y);
}
template <>
__device__ __forceinline__ void store_pair<1>(void* base, size_t idx, cf v) {
  reinterpret_cast<uint32_t*>(base)[idx / 2] = pack_bf16x2(v.x, v.y);
}

// The dispatcher hands consecutive workgroup ids to the 8 XCDs in turn.  Map
// them so that consecutive *logical* ids share an XCD (and its L2): groups of
// one (batch, head) then meet in the same L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  if ((nblocks & 7) != 0) return bid;
  return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

}  // namespace cat
