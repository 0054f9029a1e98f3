// cat_fftconv.hip -- registry of transform geometries and the launchers of
// the spectrum, FFT-convolution, score and relayout kernels.
#include "cat_fftconv.hpp"

namespace cat {

const Entry* entries_1d_small(int* n);
const Entry* entries_1d_mid(int* n);
const Entry* entries_1d_large(int* n);
const Entry* entries_2d_small(int* n);
const Entry* entries_2d_96(int* n);
const Entry* entries_2d_vit(int* n);

namespace {

using kern::ConvFn;
using kern::ScoreFn;
using kern::SpecFn;

const Entry* find_entry(const LineGeom& g) {
  using Getter = const Entry* (*)(int*);
  static const Getter getters[] = {entries_1d_small, entries_1d_mid, entries_1d_large, entries_2d_small,
                                   entries_2d_96,    entries_2d_vit};
  for (Getter get : getters) {
    int n = 0;
    const Entry* e = get(&n);
    for (int i = 0; i < n; ++i)
      if (e[i].L1 == g.L1 && e[i].L2 == g.L2 && e[i].tw == g.twiddled) return &e[i];
  }
  return nullptr;
}

int ilog2(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

}  // namespace

bool geom_supported(const LineGeom& g) { return find_entry(g) != nullptr; }

size_t line_lds_bytes(const LineGeom& g) {
  const int P2 = g.L2 + ((g.L2 % 2 == 0) ? 1 : 0);
  const int base = g.L1 * P2;
  const int LP = base + ((2 - base % 16) + 16) % 16;
  return (size_t)LP * sizeof(float2);
}

size_t spectrum_lds_bytes(const LineGeom& g, int G) {
  const Entry* e = find_entry(g);
  const int T = e ? e->T : 1;
  return (size_t)G * line_lds_bytes(g) + (size_t)((G * T + 1) / 2) * sizeof(float2);
}

int line_threads(const LineGeom& g) {
  const Entry* e = find_entry(g);
  return e ? e->T : 0;
}

int line_split(const LineGeom& g) {
  const Entry* e = find_entry(g);
  return e ? e->S : 0;
}

hipError_t prepare_kernels(const LineGeom& g, size_t conv_lds, size_t spec_lds, size_t score_lds) {
  const Entry* e = find_entry(g);
  if (!e) return hipErrorInvalidValue;
  hipError_t err = hipSuccess;
  auto raise = [&](const void* fn, size_t bytes) {
    if (fn && bytes > 0 && err == hipSuccess)
      err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  };
  raise((const void*)e->conv_f32, conv_lds);
  raise((const void*)e->conv_bf16, conv_lds);
  raise((const void*)e->spec0, spec_lds);
  raise((const void*)e->spec1, spec_lds);
  raise((const void*)e->spec2, spec_lds);
  raise((const void*)e->score, score_lds);
  raise((const void*)e->score_bf16, score_lds);
  return err;
}

hipError_t launch_spectrum(const LineGeom& g, int mode, const SpecArgs& a, hipStream_t s, const LaunchTiming* t) {
  const Entry* e = find_entry(g);
  if (mode == 1 && !g.twiddled && g.L1 == 96 && g.L2 == 96) return launch_spec96(a, s, t);
  SpecFn fn = e ? (mode == 0 ? e->spec0 : mode == 1 ? e->spec1 : e->spec2) : nullptr;
  if (!fn) return hipErrorInvalidValue;
  SpecArgs aa = a;
  if (e->S > 1 && aa.G != 1) return hipErrorInvalidValue;  // split DFTs pair adjacent lanes
  aa.log2G = ilog2(aa.G);
  const size_t lds = spectrum_lds_bytes(g, aa.G);
  const int blocks = (aa.BH + aa.G - 1) / aa.G;
  return launch_k(fn, dim3(blocks), dim3(aa.G * e->T), lds, s, t, aa);
}

hipError_t launch_conv(const LineGeom& g, int et, const ConvArgs& a, hipStream_t s, const LaunchTiming* t) {
  const Entry* e = find_entry(g);
  ConvFn fn = e ? (et == ET_F32 ? e->conv_f32 : e->conv_bf16) : nullptr;
  if (!fn) return hipErrorInvalidValue;
  ConvArgs aa = a;
  if (e->S > 1 && aa.G != 1) return hipErrorInvalidValue;  // split DFTs pair adjacent lanes
  aa.log2G = ilog2(aa.G);
  const size_t lds = (size_t)aa.G * line_lds_bytes(g);
  const int blocks = aa.B * aa.H * aa.ng;
  return launch_k(fn, dim3(blocks), dim3(aa.G * e->T), lds, s, t, aa);
}

hipError_t launch_score_partial(const LineGeom& g, const ScoreArgs& a, hipStream_t s, const LaunchTiming* t) {
  const Entry* e = find_entry(g);
  ScoreFn fn = e ? (a.et == ET_F32 ? e->score : e->score_bf16) : nullptr;
  if (!fn || a.cg < 2 || a.cg % 2 != 0 || a.npair % (a.cg / 2) != 0) return hipErrorInvalidValue;
  if (!g.twiddled && (a.et != ET_F32 || a.cg != 2)) return hipErrorInvalidValue;  // 2D reads fp32 pair lines
  if (!g.twiddled && g.L1 == 96 && g.L2 == 96) return launch_score96(a, s, t);
  const size_t lds = 2 * line_lds_bytes(g);
  return launch_k(fn, dim3(a.BH * a.ngrp), dim3(2 * e->T), lds, s, t, a);
}

namespace {

// Sum of the 2D score partials of each (batch, head): out[bh][k] =
// sum over g of part[bh][g][k], g in order (the sum the spectrum kernel
// would otherwise form itself, with far fewer workgroups).  One complex
// value per thread.
__global__ __launch_bounds__(256) void psum_kernel(const float2* __restrict__ part, float2* __restrict__ out,
                                                   int BH, int ngrp, int L) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)BH * L) return;
  const size_t line = idx / (size_t)L, k = idx - line * (size_t)L;
  const float2* src = part + line * (size_t)ngrp * L + k;
  float2 acc = src[0];
#pragma unroll 4
  for (int g = 1; g < ngrp; ++g) {
    const float2 v = src[(size_t)g * L];
    acc.x += v.x;
    acc.y += v.y;
  }
  out[idx] = acc;
}

// zr[bh][k] = z[bh][(N - k) mod N]: the line reversed about token 0, so
// that circ(softmax(zr)) = circ(softmax(z))^T.
__global__ __launch_bounds__(256) void reverse_lines_kernel(const float* __restrict__ z, float* __restrict__ zr,
                                                            int BH, int N) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)BH * N) return;
  const size_t line = idx / (size_t)N;
  const int k = (int)(idx - line * (size_t)N);
  zr[idx] = z[line * (size_t)N + (k == 0 ? 0 : N - k)];
}

}  // namespace

hipError_t launch_reverse_lines(const float* z, float* zr, int BH, int N, hipStream_t s, const LaunchTiming* t) {
  if (BH < 1 || N < 1) return hipErrorInvalidValue;
  const size_t blocks = ((size_t)BH * N + 255) / 256;
  if (blocks > 0x7fffffffu) return hipErrorInvalidValue;
  return launch_k(reverse_lines_kernel, dim3((unsigned)blocks), dim3(256), 0, s, t, z, zr, BH, N);
}

hipError_t launch_psum(const float2* part, float2* out, int BH, int ngrp, int L, hipStream_t s,
                       const LaunchTiming* t) {
  if (BH < 1 || ngrp < 1 || L < 1) return hipErrorInvalidValue;
  const size_t total = (size_t)BH * L;
  const size_t blocks = (total + 255) / 256;
  if (blocks > 0x7fffffffu) return hipErrorInvalidValue;
  return launch_k(psum_kernel, dim3((unsigned)blocks), dim3(256), 0, s, t, part, out, BH, ngrp, L);
}

hipError_t launch_relayout(const RelayoutArgs& a, hipStream_t s, const LaunchTiming* t) {
  if (a.D % 8 != 0 || a.d % 2 != 0 || a.cg % 2 != 0 || a.d % a.cg != 0) return hipErrorInvalidValue;
  if (a.D % 64 == 0 && 64 % a.cg == 0) {
    // 64 x 64 tiles through LDS
    const size_t nb = (size_t)a.B * ((a.N + 63) / 64) * (a.D / 64);
    if (nb == 0) return hipSuccess;
    if (nb > 0x7fffffffu) return hipErrorInvalidValue;
    if (a.src_et == ET_F32)
      return launch_k(kern::relayout_tile_kernel<ET_F32, 1>, dim3((unsigned)nb), dim3(256), 0, s, t, a);
    if (a.dst_f32) return launch_k(kern::relayout_tile_kernel<ET_BF16, 1>, dim3((unsigned)nb), dim3(256), 0, s, t, a);
    return launch_k(kern::relayout_tile_kernel<ET_BF16, 0>, dim3((unsigned)nb), dim3(256), 0, s, t, a);
  }
  // otherwise one thread per 16-byte chunk of a row, 4 rows each (D % 8 == 0)
  const int VE = a.src_et == ET_F32 ? 4 : 8;
  const size_t threads = (((size_t)a.B * a.N + 3) / 4) * (size_t)(a.D / VE);
  if (threads == 0) return hipSuccess;
  const size_t nb = (threads + 255) / 256;
  if (nb > 0x7fffffffu) return hipErrorInvalidValue;
  const int blocks = (int)nb;
  if (a.src_et == ET_F32) return launch_k(kern::relayout_kernel<ET_F32, 1>, dim3(blocks), dim3(256), 0, s, t, a);
  if (a.dst_f32) return launch_k(kern::relayout_kernel<ET_BF16, 1>, dim3(blocks), dim3(256), 0, s, t, a);
  return launch_k(kern::relayout_kernel<ET_BF16, 0>, dim3(blocks), dim3(256), 0, s, t, a);
}

}  // namespace cat
