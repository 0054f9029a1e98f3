// cat_api.cpp -- the C ABI (include/cat.h): validation, plans, workspace
// layout and the launch sequences of the forward paths.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/cat.h"
#include "cat_internal.hpp"

using namespace cat;

// Output tile width of the backward's weight-gradient product (fp32
// split-K slabs).
constexpr int kDwTileN = 128;

struct cat_plan_s {
  cat_problem p;
  int d;
  int et;            // ElemType of the storage dtype
  size_t esz;        // storage bytes per element
  LineGeom geom;
  int L;
  int G;             // complex lines per transform workgroup
  int ng;            // line groups per head (d / 2 / G; mconv: 8-channel groups, d / 8)
  bool mconv;        // 1D conv on the matrix cores (L = 1024, bf16, d % 16 == 0)
  bool direct;       // 1D direct circulant product on the matrix cores (bf16, N <= 256, d % 32 == 0)
  bool longn;        // 1D N beyond one workgroup's line: three passes over HBM
  bool bconv;        // 2D square grid (32 or 96 a side), bf16: the BCCB mixing on the matrix cores
  void* d_ftab = nullptr;  // bconv: its bf16 DFT-matrix fragments; mconv: its fp16 constant table
  int logL1, logL2;  // long path: L = 2^logL1 x 2^logL2
  int cg;            // channels per group of the blocked V (2 G; 8 for mconv, 32 for direct, 2 for bconv)
  int Gs;            // lines per spectrum workgroup
  int npair, ngrp, ppg;  // 2D score partials
  float2* d_tw;      // 1D inter-pass twiddles, L entries (null in 2D)
  size_t off_V, off_z, off_Q, off_K, off_part, off_psum, off_spec, ws_bytes;
  // the CAT backward's projection gradients (1D single-workgroup lines)
  size_t off_bz, off_bV, off_bdV, off_bdz, off_bWt, off_bXt, off_bP, off_bdW;
  int Hp;  // heads padded to a whole 16-byte column chunk
  // the backward's weight-gradient branch runs on a plan-owned stream
  // (default priority), forked from and joined back to the caller's stream
  hipStream_t side = nullptr;
  hipEvent_t fork_ev = nullptr, join_ev = nullptr, pack_ev = nullptr;
  size_t off_A, off_zc, off_Az;  // long path scratch
  size_t off_A2;                 // long path: the second values transform of the score gradient
  int Kp;                        // B N rounded up to 8: the padded K of the weight-gradient product
  int ksplit_dw, kchunk_dw;      // split K of the weight-gradient product: slices, K positions per slice
  size_t off_xpart, off_kbar, off_weff;  // averaged-key logits scratch (1D)
  size_t fwd_ws_bytes;  // workspace bytes the 1D forward itself touches (a prefix of the layout)
  bool debug_sync;
  int tile_n;        // forced GEMM tile width (0: the GEMM chooses)
  int tile_m;        // forced GEMM tile rows (0: the GEMM chooses)
  int num_cu;        // compute units of the device current at plan creation
  // per-launch timing slots: ev[slot][launch][start/stop], kind[slot][launch]
  static constexpr int kSlots = 256, kMaxL = 32, kMaxK = 4;
  bool timing = false;
  hipEvent_t* ev = nullptr;
  int8_t kind_of[kSlots][kMaxL];
  int nlaunch[kSlots];
  int64_t calls = 0;
  int nk = 0;
};

namespace {

thread_local std::string g_err;

cat_status fail(cat_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

cat_status hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return CAT_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
uint16_t bf16_rne(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  x += 0x7fffu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}

// The 2D matrix-core conv's DFT fragments for a side G, bf16:
// [tile i][K step t][re, im][lane][slot s] = F[lo + 16 i][32 t + 4 grp + s % 4 + 16 (s / 4)]
// for the tiles i < G / 32 (the kernel derives the others),
// F[j][k] = exp(-2 pi i j k / G), lo = lane % 16, grp = lane / 16.
void bconv_host_table(int G, std::vector<uint16_t>& tab) {
  const int NH = G / 32, KS = G / 32;
  tab.assign(bconv_table_halfs(G), 0);
  const double two_pi = 6.283185307179586476925286766559;
  size_t o = 0;
  for (int i = 0; i < NH; ++i)
    for (int t = 0; t < KS; ++t)
      for (int plane = 0; plane < 2; ++plane)
        for (int lane = 0; lane < 64; ++lane)
          for (int sl = 0; sl < 8; ++sl) {
            const int j = lane % 16 + 16 * i, k = 32 * t + 4 * (lane / 16) + sl % 4 + 16 * (sl / 4);
            const double ang = two_pi * (double)(((long)j * k) % G) / (double)G;
            tab[o++] = bf16_rne(plane == 0 ? (float)std::cos(ang) : (float)(-std::sin(ang)));
          }
}

// The 1D matrix-core conv's constants (layout: mconv_table_halfs), fp16
// rounded to nearest from double.
void mconv_host_table(std::vector<uint16_t>& tab) {
  tab.assign(mconv_table_halfs(), 0);
  const double two_pi = 6.283185307179586476925286766559;
  for (int q = 0; q < 8; ++q)
    for (int lane = 0; lane < 64; ++lane)
      for (int sl = 0; sl < 8; ++sl) {
        const int x = (q >> 1) & 1, part = q & 1;
        const int j = lane % 16 + 16 * x, k = 4 * (lane / 16) + sl % 4 + 16 * (sl / 4);
        const bool twiddle = q >= 4;
        const int L = twiddle ? 1024 : 32;
        const double ang = two_pi * (double)(((long)j * k) % L) / (double)L;
        const double v = (part == 0 ? std::cos(ang) : -std::sin(ang)) / (twiddle ? 32.0 : 1.0);
        const _Float16 hv = (_Float16)v;
        uint16_t u;
        std::memcpy(&u, &hv, 2);
        tab[((size_t)q * 64 + lane) * 8 + sl] = u;
      }
}

size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// Split a power-of-two length into L1 x L2 with L2 | L1, as balanced as possible.
void split_pow2(int L, int* L1, int* L2) {
  int e = 0;
  while ((1 << e) < L) ++e;
  *L2 = 1 << (e / 2);
  *L1 = L / *L2;
}

cat_status check_sync(const cat_plan_s* pl, const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, what);
  if (pl->debug_sync) {
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, what);
  }
  return CAT_OK;
}

char* ws_at(void* ws, size_t off) { return reinterpret_cast<char*>(ws) + off; }

void free_events(cat_plan_s* pl) {
  if (!pl->ev) return;
  for (int i = 0; i < cat_plan_s::kSlots * cat_plan_s::kMaxL * 2; ++i)
    if (pl->ev[i]) (void)hipEventDestroy(pl->ev[i]);
  delete[] pl->ev;
  pl->ev = nullptr;
}

// Timing events of one launch of the current call (null when timing is off):
// the kernel's dispatch stamps them at its start and end.  Each launch takes
// the next pair of the call's slot and records which kernel of the path it is.
struct KernelMark {
  cat_plan_s* pl;
  int slot = -1;
  LaunchTiming lt[cat_plan_s::kMaxL];
  explicit KernelMark(cat_plan_s* p) : pl(p) {
    if (pl->timing) {
      slot = (int)(pl->calls % cat_plan_s::kSlots);
      ++pl->calls;
      pl->nlaunch[slot] = 0;
    }
  }
  const LaunchTiming* at(int k) {
    if (slot < 0 || pl->nlaunch[slot] >= cat_plan_s::kMaxL) return nullptr;
    const int i = pl->nlaunch[slot]++;
    hipEvent_t* e = pl->ev + ((size_t)slot * cat_plan_s::kMaxL + i) * 2;
    pl->kind_of[slot][i] = (int8_t)k;
    lt[i] = LaunchTiming{e[0], e[1]};
    return &lt[i];
  }
};

}  // namespace

extern "C" {

const char* cat_status_string(cat_status s) {
  switch (s) {
    case CAT_OK: return "CAT_OK";
    case CAT_ERR_INVALID_ARG: return "CAT_ERR_INVALID_ARG";
    case CAT_ERR_UNSUPPORTED: return "CAT_ERR_UNSUPPORTED";
    case CAT_ERR_HIP: return "CAT_ERR_HIP";
    case CAT_ERR_ALLOC: return "CAT_ERR_ALLOC";
    case CAT_ERR_PLAN_MISMATCH: return "CAT_ERR_PLAN_MISMATCH";
  }
  return "CAT_ERR_UNKNOWN";
}

const char* cat_last_error(void) { return g_err.c_str(); }

cat_status cat_plan_create(cat_plan* out, const cat_problem* p) {
  if (out == nullptr) return fail(CAT_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (p == nullptr) return fail(CAT_ERR_INVALID_ARG, "problem is NULL");
  if (p->kind != CAT_1D && p->kind != CAT_BCCB_2D) return fail(CAT_ERR_INVALID_ARG, "unknown kind");
  if (p->dtype != CAT_F32 && p->dtype != CAT_BF16) return fail(CAT_ERR_INVALID_ARG, "unknown dtype");
  if (p->B < 0 || p->N < 1 || p->D < 1 || p->H < 1)
    return fail(CAT_ERR_INVALID_ARG, "B must be >= 0 and N, D, H >= 1");
  if (p->D % p->H != 0) return fail(CAT_ERR_INVALID_ARG, "D must be a multiple of H");
  const int64_t d = p->D / p->H;
  if (d % 2 != 0) return fail(CAT_ERR_INVALID_ARG, "head width d = D/H must be even");
  if (p->D % 8 != 0) return fail(CAT_ERR_INVALID_ARG, "D must be a multiple of 8");
  {
    // B N D < 2^31 and B H <= 2^24, tested without forming an overflowing product
    const int64_t lim = (int64_t(1) << 31) - 1;
    const bool big = p->N > lim || p->D > lim || p->N * p->D > lim || p->B > lim / (p->N * p->D) ||
                     p->B > (int64_t(1) << 24) / p->H;
    if (big) return fail(CAT_ERR_UNSUPPORTED, "problem too large (B*N*D must be < 2^31)");
  }

  if (p->kind == CAT_1D && p->H > 32)
    return fail(CAT_ERR_UNSUPPORTED, "1D supports at most 32 heads (score projection fused into the GEMM)");

  LineGeom g{};
  // beyond one workgroup's line: a power-of-two N up to 65536 (L = N), or
  // any other N up to 32768 on the power-of-two circle L >= 2N - 1
  const bool longn = p->kind == CAT_1D && ((is_pow2(p->N) && p->N > 4096 && p->N <= 65536) ||
                                           (!is_pow2(p->N) && p->N > 2048 && p->N <= 32768));
  if (longn) {
    // three passes over HBM, L = L1 x L2 (L1 >= L2)
    const int64_t Lmin = is_pow2(p->N) ? p->N : 2 * p->N - 1;
    int e = 0;
    while ((int64_t(1) << e) < Lmin) ++e;
    g.L1 = 1 << ((e + 1) / 2);
    g.L2 = 1 << (e / 2);
    g.twiddled = 1;
  } else if (p->kind == CAT_1D) {
    int L = 0;
    if (is_pow2(p->N) && p->N <= 4096) {
      L = (int)p->N;
    } else if (2 * p->N - 1 <= 4096) {
      L = 1;
      while (L < 2 * p->N - 1) L <<= 1;
    } else {
      return fail(CAT_ERR_UNSUPPORTED,
                  "1D N beyond the supported lengths (powers of two up to 65536, other N up to 32768)");
    }
    split_pow2(L, &g.L1, &g.L2);
    g.twiddled = 1;
  } else {
    if (p->Hg < 1 || p->Wg < 1 || p->Hg * p->Wg != p->N)
      return fail(CAT_ERR_INVALID_ARG, "2D needs Hg, Wg >= 1 and Hg*Wg == N");
    g.L1 = (int)p->Hg;
    g.L2 = (int)p->Wg;
    g.twiddled = 0;
  }
  if (!longn && !geom_supported(g)) return fail(CAT_ERR_UNSUPPORTED, "transform length / grid not instantiated");

  cat_plan_s* pl = new (std::nothrow) cat_plan_s();
  if (!pl) return fail(CAT_ERR_ALLOC, "host allocation failed");
  pl->p = *p;
  pl->d = (int)d;
  pl->et = p->dtype == CAT_F32 ? ET_F32 : ET_BF16;
  pl->esz = p->dtype == CAT_F32 ? 4 : 2;
  pl->geom = g;
  pl->L = g.L1 * g.L2;
  pl->longn = longn;
  pl->logL1 = pl->logL2 = 0;
  while ((1 << pl->logL1) < g.L1) ++pl->logL1;
  while ((1 << pl->logL2) < g.L2) ++pl->logL2;
  const int T = longn ? 1 : line_threads(g);
  const size_t line_bytes = longn ? 0 : line_lds_bytes(g);
  const int d2 = (int)d / 2;
  // lines per transform workgroup: power of two dividing d/2, <= 256 threads
  // (the long path instead takes pair blocks: the largest power of two <= 8 dividing d/2)
  int G = 1;
  const size_t lds_cap = p->kind == CAT_1D ? 96 * 1024 : 152 * 1024;
  if (longn)
    while (G < 8 && d2 % (2 * G) == 0) G *= 2;
  else
    // (split DFTs pair lanes of one line: one line per workgroup)
    while (line_split(g) == 1 && G < 8 && d2 % (2 * G) == 0 && (2 * G) * T <= 256 && (2 * G) * line_bytes <= lds_cap)
      G *= 2;
  {
    const char* cv = std::getenv("CAT_CONV");
    const bool force_valu = cv && std::strcmp(cv, "valu") == 0;
    const bool force_fft = force_valu || (cv && std::strcmp(cv, "fft") == 0);
    pl->direct = !force_fft && p->kind == CAT_1D && p->dtype == CAT_BF16 && p->N <= 256 && d % 32 == 0;
    pl->mconv = !longn && !pl->direct && !force_valu && p->kind == CAT_1D && p->dtype == CAT_BF16 &&
                g.L1 * g.L2 == 1024 && d % 16 == 0;
    pl->bconv = !force_valu && p->kind == CAT_BCCB_2D && p->dtype == CAT_BF16 && p->Hg == p->Wg &&
                bconv_supported((int)p->Hg) && d % 8 == 0;
    pl->G = G;
    pl->ng = d2 / G;
    pl->cg = pl->direct ? 32 : pl->mconv ? 8 : pl->bconv ? 2 : 2 * G;
    if (pl->mconv) pl->ng = (int)d / 8;
    if (pl->direct) pl->ng = (int)d / 32;
  }
  int Gs = 1;
  while ((2 * Gs) * T <= 64 && spectrum_lds_bytes(g, 2 * Gs) <= 96 * 1024) Gs *= 2;
  pl->Gs = Gs;
  pl->npair = d2;
  // pairs per score workgroup: 2 -- at the 96x96 workload (48 heads x 32
  // pairs) that is 768 workgroups of one per CU, three even rounds on 256
  // CUs; with 4 it was 384, and half the CUs ran two
  pl->ppg = 2;
  pl->ngrp = (d2 + pl->ppg - 1) / pl->ppg;
  const char* ds = std::getenv("CAT_DEBUG_SYNC");
  pl->debug_sync = ds && ds[0] == '1';
  const char* tn = std::getenv("CAT_GEMM_TILE_N");
  pl->tile_n = tn ? std::atoi(tn) : 0;
  if (pl->tile_n != 96 && pl->tile_n != 128 && pl->tile_n != 192) pl->tile_n = 0;
  const char* tm = std::getenv("CAT_GEMM_TILE_M");
  pl->tile_m = tm ? std::atoi(tm) : 0;
  if (pl->tile_m != 128 && pl->tile_m != 256) pl->tile_m = 0;

  {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      n = 0;
    pl->num_cu = n;
  }
  const size_t BND = (size_t)p->B * p->N * p->D;
  const size_t BH = (size_t)p->B * p->H;
  size_t off = 0;
  pl->off_V = off;
  off = up256(off + BND * pl->esz);
  pl->off_spec = off;
  off = up256(off + BH * pl->L * sizeof(float2));
  pl->off_A = pl->off_zc = pl->off_Az = 0;
  if (p->kind == CAT_1D) {
    pl->off_z = off;
    off = up256(off + BH * p->N * sizeof(float));
    pl->off_Q = pl->off_K = pl->off_part = pl->off_psum = pl->off_A2 = 0;
    pl->fwd_ws_bytes = off;  // V, spectrum, logits (the long path adds its scratch below)
    if (longn) {
      pl->off_A = off;
      off = up256(off + BH * (size_t)d2 * pl->L * sizeof(float2));
      pl->off_zc = off;
      off = up256(off + BH * pl->L * sizeof(float2));
      pl->off_Az = off;
      off = up256(off + BH * pl->L * sizeof(float2));
      pl->fwd_ws_bytes = off;
    }
    // the mixing backward: V in the blocked layout, then the score-gradient
    // partials and their sum (single-workgroup lines) or the second values
    // transform (the long path, whose cross-spectrum line reuses Az and
    // whose correlation line reuses zc)
    pl->off_Q = off;
    off = up256(off + BND * pl->esz);
    if (!longn) {
      pl->off_part = off;
      off = up256(off + BH * pl->ngrp * pl->L * sizeof(float2));
      pl->off_psum = off;
      off = up256(off + BH * pl->L * sizeof(float2));
    } else {
      pl->off_A2 = off;
      off = up256(off + BH * (size_t)d2 * pl->L * sizeof(float2));
    }
    // the whole backward: V and z recomputed, dV and dz, [W_V^T ; W_A^T ; 0],
    // X^T (B N padded to Kp columns), P = [dV | dz^T | 0] (dz padded to Hp
    // heads) and the split-K partial products of [dW_V | dW_A | 0] (fp32)
    {
      const size_t Dz = (size_t)p->D, BN = (size_t)p->B * p->N;
      pl->Hp = (int)((p->H + 7) / 8 * 8);
      pl->Kp = (int)((BN + 7) / 8 * 8);
      // K = B N is long and the output only D x (D + Hp): slices of K fill
      // one round of two workgroups per compute unit with kDwTileN-wide
      // tiles (at least 512 K positions per slice, a multiple of the K tile)
      {
        const long cus = pl->num_cu > 0 ? pl->num_cu : 256;
        const long tiles = ((long)p->D + 127) / 128 * (((long)p->D + pl->Hp + kDwTileN - 1) / kDwTileN);
        const long kt = pl->esz == 4 ? 32 : 64;
        long S = 2 * cus / tiles;
        const long smax = (long)BN / 512;
        S = S < smax ? S : smax;
        S = S < 1 ? 1 : S;
        long kc = ((long)BN + S - 1) / S;
        kc = kc < 1 ? kt : (kc + kt - 1) / kt * kt;  // (an empty batch: one slice of one K tile)
        pl->kchunk_dw = (int)kc;
        pl->ksplit_dw = BN == 0 ? 1 : (int)(((long)BN + kc - 1) / kc);
      }
      const size_t sizes[8] = {BH * p->N * sizeof(float), BND * pl->esz, BND * pl->esz, BH * p->N * sizeof(float),
                               (Dz + pl->Hp) * Dz * pl->esz, Dz * (size_t)pl->Kp * pl->esz,
                               BN * (Dz + pl->Hp) * pl->esz,
                               (size_t)pl->ksplit_dw * Dz * (Dz + pl->Hp) * sizeof(float)};
      size_t* offs[8] = {&pl->off_bz, &pl->off_bV, &pl->off_bdV, &pl->off_bdz, &pl->off_bWt,
                         &pl->off_bXt, &pl->off_bP, &pl->off_bdW};
      for (int i = 0; i < 8; ++i) {
        *offs[i] = off;
        off = up256(off + sizes[i]);
      }
    }
    // the averaged-key logits: column-sum partials, mean key, score weights
    pl->off_xpart = off;
    off = up256(off + avgkey_part_floats((int)p->B, (int)p->N, (int)p->D) * sizeof(float));
    pl->off_kbar = off;
    off = up256(off + (size_t)p->B * p->D * sizeof(float));
    pl->off_weff = off;
    off = up256(off + (size_t)p->B * p->D * p->H * sizeof(float));
  } else {
    pl->fwd_ws_bytes = 0;  // (1D only)
    pl->off_z = off;  // the CAT-scored variant's logits
    off = up256(off + BH * p->N * sizeof(float));
    pl->off_Q = off;
    off = up256(off + BND * sizeof(float));
    pl->off_K = off;
    off = up256(off + BND * sizeof(float));
    pl->off_part = off;
    off = up256(off + BH * pl->ngrp * pl->L * sizeof(float2));
    pl->off_psum = off;
    off = up256(off + BH * pl->L * sizeof(float2));
  }
  pl->ws_bytes = off;

  // device tables and kernel attributes
  pl->d_tw = nullptr;
  if (g.twiddled) {
    std::vector<float2> tw((size_t)pl->L);
    const double two_pi = 6.283185307179586476925286766559;
    if (longn) {
      // long path: W_L^m for every m < L
      for (int m = 0; m < pl->L; ++m) {
        const double ang = two_pi * (double)m / (double)pl->L;
        tw[(size_t)m] = make_float2((float)std::cos(ang), (float)(-std::sin(ang)));
      }
    } else {
      for (int n2 = 0; n2 < g.L2; ++n2)
        for (int k1 = 0; k1 < g.L1; ++k1) {
          const long e = ((long)n2 * k1) % pl->L;
          const double ang = two_pi * (double)e / (double)pl->L;
          tw[(size_t)k1 * g.L2 + n2] = make_float2((float)std::cos(ang), (float)(-std::sin(ang)));
        }
    }
    hipError_t e = hipMalloc(&pl->d_tw, tw.size() * sizeof(float2));
    if (e != hipSuccess) {
      delete pl;
      return hip_fail(e, "hipMalloc(twiddles)");
    }
    e = hipMemcpy(pl->d_tw, tw.data(), tw.size() * sizeof(float2), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(pl->d_tw);
      delete pl;
      return hip_fail(e, "hipMemcpy(twiddles)");
    }
  }
  if (pl->bconv || pl->mconv) {
    std::vector<uint16_t> tab;
    if (pl->bconv) bconv_host_table((int)p->Hg, tab);
    else mconv_host_table(tab);
    hipError_t e = hipMalloc(&pl->d_ftab, tab.size() * sizeof(uint16_t));
    if (e == hipSuccess) e = hipMemcpy(pl->d_ftab, tab.data(), tab.size() * sizeof(uint16_t), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      if (pl->d_ftab) (void)hipFree(pl->d_ftab);
      if (pl->d_tw) (void)hipFree(pl->d_tw);
      delete pl;
      return hip_fail(e, "DFT table upload");
    }
  }
  hipError_t e = longn ? hipSuccess : prepare_kernels(g, (size_t)G * line_bytes, spectrum_lds_bytes(g, Gs), 2 * line_bytes);
  if (e != hipSuccess) {
    if (pl->d_tw) (void)hipFree(pl->d_tw);
    if (pl->d_ftab) (void)hipFree(pl->d_ftab);
    delete pl;
    return hip_fail(e, "hipFuncSetAttribute");
  }


  if (p->kind == CAT_1D) {  // the backward's weight-gradient branch
    hipError_t se = hipStreamCreateWithFlags(&pl->side, hipStreamNonBlocking);
    if (se == hipSuccess) se = hipEventCreateWithFlags(&pl->fork_ev, hipEventDisableTiming);
    if (se == hipSuccess) se = hipEventCreateWithFlags(&pl->join_ev, hipEventDisableTiming);
    if (se == hipSuccess) se = hipEventCreateWithFlags(&pl->pack_ev, hipEventDisableTiming);
    if (se != hipSuccess) {
      if (pl->join_ev) (void)hipEventDestroy(pl->join_ev);
      if (pl->fork_ev) (void)hipEventDestroy(pl->fork_ev);
      if (pl->side) (void)hipStreamDestroy(pl->side);
      if (pl->d_tw) (void)hipFree(pl->d_tw);
      if (pl->d_ftab) (void)hipFree(pl->d_ftab);
      delete pl;
      return hip_fail(se, "stream / event creation");
    }
  }

  *out = pl;
  g_err.clear();
  return CAT_OK;
}

cat_status cat_plan_destroy(cat_plan plan) {
  if (plan == nullptr) return CAT_OK;
  if (plan->d_tw) (void)hipFree(plan->d_tw);
  if (plan->d_ftab) (void)hipFree(plan->d_ftab);
  free_events(plan);
  if (plan->pack_ev) (void)hipEventDestroy(plan->pack_ev);
  if (plan->join_ev) (void)hipEventDestroy(plan->join_ev);
  if (plan->fork_ev) (void)hipEventDestroy(plan->fork_ev);
  if (plan->side) (void)hipStreamDestroy(plan->side);

  delete plan;
  return CAT_OK;
}

cat_status cat_plan_set_timing(cat_plan plan, int enable) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  plan->timing = false;
  plan->calls = 0;
  if (!enable) return CAT_OK;
  if (!plan->ev) {
    const int n = cat_plan_s::kSlots * cat_plan_s::kMaxL * 2;
    plan->ev = new (std::nothrow) hipEvent_t[n]();
    if (!plan->ev) return fail(CAT_ERR_ALLOC, "event table allocation failed");
    for (int i = 0; i < n; ++i) {
      hipError_t e = hipEventCreate(&plan->ev[i]);
      if (e != hipSuccess) {
        free_events(plan);
        return hip_fail(e, "hipEventCreate");
      }
    }
  }
  plan->timing = true;
  return CAT_OK;
}

cat_status cat_plan_kernel_times(cat_plan plan, double* total_ms, int64_t* launches, int* nkernels) {
  if (!plan || !total_ms || !launches || !nkernels) return fail(CAT_ERR_INVALID_ARG, "NULL argument");
  const int nk = plan->p.kind == CAT_1D ? 9 : 5;
  *nkernels = nk;
  for (int k = 0; k < 16; ++k) {
    total_ms[k] = 0.0;
    launches[k] = 0;
  }
  if (!plan->ev || plan->calls == 0) return CAT_OK;
  const int64_t n = plan->calls < cat_plan_s::kSlots ? plan->calls : cat_plan_s::kSlots;
  for (int64_t c = 0; c < n; ++c) {
    for (int i = 0; i < plan->nlaunch[c]; ++i) {
      hipEvent_t* e = plan->ev + ((size_t)c * cat_plan_s::kMaxL + i) * 2;
      hipError_t err = hipEventSynchronize(e[1]);
      if (err != hipSuccess) return hip_fail(err, "hipEventSynchronize");
      float ms = 0.f;
      err = hipEventElapsedTime(&ms, e[0], e[1]);
      if (err != hipSuccess) return hip_fail(err, "hipEventElapsedTime");
      const int k = plan->kind_of[c][i];
      total_ms[k] += ms;
      launches[k] += 1;
    }
  }
  return CAT_OK;
}

cat_status cat_plan_workspace_size(cat_plan plan, size_t* bytes) {
  if (!plan || !bytes) return fail(CAT_ERR_INVALID_ARG, "NULL argument");
  *bytes = plan->ws_bytes;
  return CAT_OK;
}

cat_status cat_plan_conv_path(cat_plan plan, int* path) {
  if (!plan || !path) return fail(CAT_ERR_INVALID_ARG, "NULL argument");
  *path = plan->longn ? CAT_PATH_FFT_MULTIPASS
         : plan->direct ? CAT_PATH_DIRECT
         : (plan->mconv || plan->bconv) ? CAT_PATH_FFT_MATRIX
                        : CAT_PATH_FFT_VALU;
  return CAT_OK;
}

cat_status cat_plan_geometry(cat_plan plan, int64_t* L, int64_t* L1, int64_t* L2) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  if (L) *L = plan->L;
  if (L1) *L1 = plan->geom.L1;
  if (L2) *L2 = plan->geom.L2;
  return CAT_OK;
}

}  // extern "C"

namespace {

cat_status check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* q : ps) {
    if (q == nullptr) return fail(CAT_ERR_INVALID_ARG, "NULL buffer");
    if (!aligned16(q)) return fail(CAT_ERR_INVALID_ARG, "buffer not 16-byte aligned");
  }
  return CAT_OK;
}

GemmArgs gemm_base(const cat_plan_s* pl, const void* X) {
  GemmArgs a{};
  a.X = X;
  a.M = (int)(pl->p.B * pl->p.N);
  a.K = (int)pl->p.D;
  a.Ntok = (int)pl->p.N;
  a.H = (int)pl->p.H;
  a.d = pl->d;
  a.num_cu = pl->num_cu;
  a.tile_n = pl->tile_n;
  a.tile_m = pl->tile_m;
  return a;
}

GemmSeg seg(const void* W, void* out, int ncols, int out_f32, int layout, int cg) {
  GemmSeg s{};
  s.W = W;
  s.out = out;
  s.ncols = ncols;
  s.out_f32 = out_f32;
  s.layout = layout;
  s.cg = cg;
  return s;
}

SpecArgs spec_base(const cat_plan_s* pl, void* ws) {
  SpecArgs a{};
  a.spec = reinterpret_cast<float2*>(ws_at(ws, pl->off_spec));
  a.tw = pl->d_tw;
  a.BH = (int)(pl->p.B * pl->p.H);
  a.N = (int)pl->p.N;
  a.scale = 1.0f;
  a.G = pl->Gs;
  a.transpose = pl->bconv ? 1 : 0;  // the 2D matrix-core conv reads S with kc contiguous
  return a;
}

ConvArgs conv_base(const cat_plan_s* pl, const void* Vblk, const float2* spec, void* O) {
  ConvArgs a{};
  a.V = Vblk;
  a.spec = spec;
  a.tw = pl->d_tw;
  a.O = O;
  a.B = (int)pl->p.B;
  a.H = (int)pl->p.H;
  a.D = (int)pl->p.D;
  a.N = (int)pl->p.N;
  a.d = pl->d;
  a.G = pl->G;
  a.ng = pl->ng;
  a.mtab = pl->mconv ? pl->d_ftab : nullptr;
  return a;
}

LongArgs long_base(const cat_plan_s* pl) {
  LongArgs a{};
  a.tw = pl->d_tw;
  a.logL1 = pl->logL1;
  a.logL2 = pl->logL2;
  a.BH = (int)(pl->p.B * pl->p.H);
  a.pairs = pl->d / 2;
  a.N = (int)pl->p.N;
  a.H = (int)pl->p.H;
  a.D = (int)pl->p.D;
  a.d = pl->d;
  a.pb = pl->cg / 2;
  return a;
}

// The long-sequence mixing (three passes): softmax line and filter spectrum
// (timing slot 1), then the values (slot 2).
hipError_t run_long_1d(const cat_plan_s* pl, const float* logits, const void* Vb, void* O, void* ws, hipStream_t s,
                       KernelMark* mk) {
  const LaunchTiming* ts[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  if (mk) {
    for (int i = 0; i < 3; ++i) ts[i] = mk->at(1);
    for (int i = 3; i < 6; ++i) ts[i] = mk->at(2);
  }
  return launch_longconv(pl->et, long_base(pl), logits, Vb, reinterpret_cast<float2*>(ws_at(ws, pl->off_zc)),
                         reinterpret_cast<float2*>(ws_at(ws, pl->off_Az)),
                         reinterpret_cast<float2*>(ws_at(ws, pl->off_spec)),
                         reinterpret_cast<float2*>(ws_at(ws, pl->off_A)), O, s, ts);
}

// The conv of a plan's path (1D: matrix-core FFT, direct product or vector
// FFT; 2D: matrix-core or vector FFT) from V in the plan's blocked layout.
hipError_t run_conv_1d(const cat_plan_s* pl, const ConvArgs& ca, hipStream_t s, const LaunchTiming* t = nullptr) {
  if (pl->direct) return launch_dconv(pl->et, ca, s, t);
  if (pl->bconv) {
    BconvArgs b{};
    b.V = ca.V;
    b.spec = ca.spec;
    b.table = pl->d_ftab;
    b.O = ca.O;
    b.BH = ca.B * ca.H;
    b.npair = ca.d / 2;
    b.H = ca.H;
    b.D = ca.D;
    b.d = ca.d;
    b.num_cu = pl->num_cu;
    return launch_bconv(b, (int)pl->p.Hg, s, t);
  }
  return pl->mconv ? launch_mconv(ca, s, t) : launch_conv(pl->geom, pl->et, ca, s, t);
}

// The mixing O = circ(softmax(logits)) V (1D) or BCCB(..) V (2D) from
// [B][N][D] values: relayout to the blocked layout, then the plan's path.
cat_status mix_impl(cat_plan plan, const float* logits, const void* V, void* O, void* workspace, hipStream_t s,
                    KernelMark* mk = nullptr) {
  cat_status st = CAT_OK;
  void* Vb = ws_at(workspace, plan->off_V);
  RelayoutArgs ra{};
  ra.src = V;
  ra.dst = Vb;
  ra.src_et = plan->et;
  ra.dst_f32 = 0;
  ra.B = (int)plan->p.B;
  ra.N = (int)plan->p.N;
  ra.D = (int)plan->p.D;
  ra.H = (int)plan->p.H;
  ra.d = plan->d;
  ra.cg = plan->cg;
  hipError_t e = launch_relayout(ra, s, mk ? mk->at(4) : nullptr);
  if (e != hipSuccess) return hip_fail(e, "relayout launch");
  if (plan->longn) {
    e = run_long_1d(plan, logits, Vb, O, workspace, s, mk);
    if (e != hipSuccess) return hip_fail(e, "long-sequence fft-conv launch");
    return check_sync(plan, "long-sequence fft-conv");
  }
  SpecArgs sa = spec_base(plan, workspace);
  sa.logits = logits;
  const bool own_softmax = plan->mconv || plan->direct;
  if (!own_softmax) {
    e = launch_spectrum(plan->geom, 0, sa, s, mk ? mk->at(1) : nullptr);
    if (e != hipSuccess) return hip_fail(e, "spectrum launch");
    if ((st = check_sync(plan, "spectrum")) != CAT_OK) return st;
  }
  ConvArgs ca = conv_base(plan, Vb, sa.spec, O);
  if (own_softmax) ca.logits = logits;
  e = run_conv_1d(plan, ca, s, mk ? mk->at(2) : nullptr);
  if (e != hipSuccess) return hip_fail(e, "fft-conv launch");
  return check_sync(plan, "fft-conv");
}


const LaunchTiming* mk_at(KernelMark* mk, int k) { return mk ? mk->at(k) : nullptr; }

// The mixing backward (see cat_step_mix_backward_1d), plan and pointers checked.
cat_status mix_backward_core(cat_plan plan, const float* logits, const void* V, const void* dO, float* dlogits,
                             void* dV, void* workspace, hipStream_t s, KernelMark* mk) {
  cat_status st = CAT_OK;
  const int BH = (int)(plan->p.B * plan->p.H), N = (int)plan->p.N;
  // dV = circ(z*)^T dO = circ(softmax(zr)) dO with zr the reversed logits
  float* zr = reinterpret_cast<float*>(ws_at(workspace, plan->off_z));
  hipError_t e = launch_reverse_lines(logits, zr, BH, N, s, mk_at(mk, 3));
  if (e != hipSuccess) return hip_fail(e, "reverse launch");
  if ((st = mix_impl(plan, zr, dO, dV, workspace, s, mk)) != CAT_OK) return st;
  // dz*: cross-correlation spectra of dO and V per pair group, summed per
  // (batch, head).  dO is still in the workspace in the blocked layout the
  // dV mixing made of it; V gets the same layout.
  const void* dOb = ws_at(workspace, plan->off_V);
  void* Vb = ws_at(workspace, plan->off_Q);
  float2* part = reinterpret_cast<float2*>(ws_at(workspace, plan->off_part));
  float2* psum = reinterpret_cast<float2*>(ws_at(workspace, plan->off_psum));
  RelayoutArgs ra{};
  ra.src = V;
  ra.dst = Vb;
  ra.src_et = plan->et;
  ra.dst_f32 = 0;
  ra.B = (int)plan->p.B;
  ra.N = N;
  ra.D = (int)plan->p.D;
  ra.H = (int)plan->p.H;
  ra.d = plan->d;
  ra.cg = plan->cg;
  if ((e = launch_relayout(ra, s, mk_at(mk, 4))) != hipSuccess) return hip_fail(e, "relayout launch");
  if (plan->longn) {
    // the cross-correlation spectra of every pair of a head summed before
    // one inverse transform (three passes), then dlogits
    e = launch_long_scoregrad(plan->et, long_base(plan), logits, dOb, Vb,
                              reinterpret_cast<float2*>(ws_at(workspace, plan->off_A)),
                              reinterpret_cast<float2*>(ws_at(workspace, plan->off_A2)),
                              reinterpret_cast<float2*>(ws_at(workspace, plan->off_Az)),
                              reinterpret_cast<float*>(ws_at(workspace, plan->off_zc)), dlogits, s, mk_at(mk, 5));
    if (e != hipSuccess) return hip_fail(e, "long score-gradient launch");
    return check_sync(plan, "mixing backward");
  }
  ScoreArgs sc{};
  sc.Q = dOb;
  sc.K = Vb;
  sc.et = plan->et;
  sc.cg = plan->cg;
  sc.partial = part;
  sc.BH = BH;
  sc.N = N;
  sc.npair = plan->npair;
  sc.ngrp = plan->ngrp;
  sc.ppg = plan->ppg;
  sc.tw = plan->d_tw;
  if ((e = launch_score_partial(plan->geom, sc, s, mk_at(mk, 5))) != hipSuccess)
    return hip_fail(e, "score-gradient launch");
  if ((e = launch_psum(part, psum, BH, plan->ngrp, plan->L, s, mk_at(mk, 6))) != hipSuccess)
    return hip_fail(e, "psum launch");
  // dlogits = z* (dz* - <z*, dz*>)
  SpecArgs sa = spec_base(plan, workspace);
  sa.logits = logits;
  sa.partial = psum;
  sa.ngrp = 1;
  sa.probs = dlogits;
  if ((e = launch_spectrum(plan->geom, 2, sa, s, mk_at(mk, 7))) != hipSuccess)
    return hip_fail(e, "logits-gradient launch");
  return check_sync(plan, "mixing backward");
}

// The whole backward after the fork (the plan's side stream already waits
// for `s`).  With P = [dV | dz^T | 0] [B N][D + Hp] (storage dtype):
//   side stream: X^T (needs only X, so it runs beside the projection and
//                the mixing backward), then, once P is packed,
//                [dW_V | dW_A | 0] = X^T P with K split into slices whose
//                fp32 partial products are summed in order;
//   `s`:         V and z recomputed, the mixing backward (dV, dz), P, then
//                dX = P [W_V^T ; W_A^T ; 0] (K = D + Hp), written in the
//                storage dtype from fp32 accumulators.
// Returns the first failure; the caller joins the side stream either way.
cat_status backward_body(cat_plan plan, const void* X, const void* W_A, const void* W_V, const void* dO, void* dX,
                         void* dW_A, void* dW_V, void* workspace, hipStream_t s, KernelMark* mk) {
  const int B = (int)plan->p.B, N = (int)plan->p.N, D = (int)plan->p.D, H = (int)plan->p.H, Hp = plan->Hp;
  const int et = plan->et;
  hipError_t e;
  cat_status st;
  hipStream_t sw = plan->side;
  void* bXt = ws_at(workspace, plan->off_bXt);
  if ((e = launch_transpose(et, X, bXt, B * N, D, plan->Kp, sw)) != hipSuccess) return hip_fail(e, "transpose launch");

  // the forward's V (row-major) and logits
  void* bV = ws_at(workspace, plan->off_bV);
  float* bz = reinterpret_cast<float*>(ws_at(workspace, plan->off_bz));
  void* bdV = ws_at(workspace, plan->off_bdV);
  float* bdz = reinterpret_cast<float*>(ws_at(workspace, plan->off_bdz));
  GemmArgs ga = gemm_base(plan, X);
  ga.nseg = 1;
  ga.seg[0] = seg(W_V, bV, D, 0, OUT_ROWMAJOR, 1);
  ga.Wz = W_A;
  ga.z = bz;
  ga.nz = H;
  if ((e = launch_gemm(et, ga, s, mk->at(0))) != hipSuccess) return hip_fail(e, "projection launch");
  // dlogits (fp32) and dV
  if ((st = mix_backward_core(plan, bz, bV, dO, bdz, bdV, workspace, s, mk)) != CAT_OK) return st;
  void* P = ws_at(workspace, plan->off_bP);
  if ((e = launch_pack_grads(et, bdV, bdz, P, B, N, D, H, Hp, s)) != hipSuccess) return hip_fail(e, "pack launch");
  if ((e = hipEventRecord(plan->pack_ev, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if ((e = hipStreamWaitEvent(sw, plan->pack_ev, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");

  // weight gradients (side stream)
  const int S = plan->ksplit_dw;
  float* pW = reinterpret_cast<float*>(ws_at(workspace, plan->off_bdW));  // [S][D][D + Hp] fp32
  GemmArgs gw = gemm_base(plan, bXt);
  gw.M = D;
  gw.K = B * N;
  gw.ldx = plan->Kp;  // X^T rows padded to 16-byte multiples (zero past B N)
  gw.ksplit = S;      // slices of K, each writing fp32 partial products
  gw.kchunk = plan->kchunk_dw;
  gw.tile_n = plan->tile_n ? plan->tile_n : kDwTileN;
  gw.nseg = 1;
  gw.seg[0] = seg(P, pW, D + Hp, 1, OUT_ROWMAJOR, 1);
  if ((e = launch_gemm(et, gw, sw)) != hipSuccess) return hip_fail(e, "dW launch");
  if ((e = launch_sum_slices(et, pW, dW_V, dW_A, S, D, D + Hp, D, H, sw)) != hipSuccess)
    return hip_fail(e, "dW sum launch");

  // dX (s): Wc = [W_V^T ; W_A^T ; 0] [D + Hp][D]
  char* Wc = reinterpret_cast<char*>(ws_at(workspace, plan->off_bWt));
  if ((e = launch_transpose(et, W_V, Wc, D, D, D, s)) != hipSuccess) return hip_fail(e, "transpose launch");
  if ((e = launch_transpose(et, W_A, Wc + (size_t)D * D * plan->esz, D, H, D, s)) != hipSuccess)
    return hip_fail(e, "transpose launch");
  if ((e = launch_zero(Wc + (size_t)(D + H) * D * plan->esz, (size_t)(Hp - H) * D * plan->esz, s)) != hipSuccess)
    return hip_fail(e, "zero launch");
  GemmArgs gx = gemm_base(plan, P);
  gx.K = D + Hp;
  gx.nseg = 1;
  gx.seg[0] = seg(Wc, dX, D, 0, OUT_ROWMAJOR, 1);
  if ((e = launch_gemm(et, gx, s)) != hipSuccess) return hip_fail(e, "dX launch");
  return CAT_OK;
}

// Join: `s` waits for everything queued on the plan's side stream.
cat_status join_side(cat_plan plan, hipStream_t s) {
  hipError_t e = hipEventRecord(plan->join_ev, plan->side);
  if (e != hipSuccess) {
    // without the event, wait for the side stream from the host instead
    (void)hipStreamSynchronize(plan->side);
    return hip_fail(e, "hipEventRecord");
  }
  if ((e = hipStreamWaitEvent(s, plan->join_ev, 0)) != hipSuccess) {
    (void)hipStreamSynchronize(plan->side);
    return hip_fail(e, "hipStreamWaitEvent");
  }
  return CAT_OK;
}

// The 1D mixing from logits z [B][H][N] and V already in the blocked
// layout of the plan's path (plan->cg channels per group): the plan's path
// (matrix-core FFT, direct product, vector FFT or the three passes).
cat_status mix_from_blocked(cat_plan plan, const float* z, const void* Vb, void* O, void* workspace, hipStream_t s,
                            KernelMark* mk) {
  hipError_t e;
  cat_status st;
  if (plan->longn) {
    e = run_long_1d(plan, z, Vb, O, workspace, s, mk);
    if (e != hipSuccess) return hip_fail(e, "long-sequence fft-conv launch");
    return check_sync(plan, "long-sequence fft-conv");
  }
  SpecArgs sa = spec_base(plan, workspace);
  sa.logits = z;
  const bool own_softmax = plan->mconv || plan->direct;  // (these take the logits themselves)
  if (!own_softmax) {
    e = launch_spectrum(plan->geom, 0, sa, s, mk_at(mk, 1));
    if (e != hipSuccess) return hip_fail(e, "spectrum launch");
    if ((st = check_sync(plan, "spectrum")) != CAT_OK) return st;
  }
  ConvArgs ca = conv_base(plan, Vb, sa.spec, O);
  if (own_softmax) ca.logits = z;
  e = run_conv_1d(plan, ca, s, mk_at(mk, 2));
  if (e != hipSuccess) return hip_fail(e, "fft-conv launch");
  return check_sync(plan, "fft-conv");
}

cat_status avgkey_supported(const cat_plan_s* pl) {
  if (pl->p.D > 3072)
    return fail(CAT_ERR_UNSUPPORTED, "the averaged-key logits support D <= 3072");
  if (pl->p.B > 65535) return fail(CAT_ERR_UNSUPPORTED, "the averaged-key logits support B <= 65535");
  return CAT_OK;
}

// Averaged-key logits into z (timing slots: kind 8).
cat_status avgkey_logits(cat_plan plan, const void* X, const void* W_Q, const void* W_K, float* z, void* workspace,
                         hipStream_t s, KernelMark* mk) {
  AvgKeyArgs a{};
  a.X = X;
  a.W_Q = W_Q;
  a.W_K = W_K;
  a.part = reinterpret_cast<float*>(ws_at(workspace, plan->off_xpart));
  a.kbar = reinterpret_cast<float*>(ws_at(workspace, plan->off_kbar));
  a.weff = reinterpret_cast<float*>(ws_at(workspace, plan->off_weff));
  a.z = z;
  a.B = (int)plan->p.B;
  a.N = (int)plan->p.N;
  a.D = (int)plan->p.D;
  a.H = (int)plan->p.H;
  a.scale = 1.0f / std::sqrt((float)plan->d);
  const LaunchTiming* ts[5] = {mk_at(mk, 8), mk_at(mk, 8), mk_at(mk, 8), mk_at(mk, 8), mk_at(mk, 8)};
  hipError_t e = launch_avgkey(plan->et, a, s, ts);
  if (e != hipSuccess) return hip_fail(e, "averaged-key logits launch");
  return check_sync(plan, "averaged-key logits");
}

// Causal CAT runs on the direct product: bf16, N <= 256, 32-channel groups.
constexpr int kCausalCg = 32;
cat_status causal_supported(const cat_plan_s* pl) {
  if (pl->et != ET_BF16 || pl->p.N > 256 || pl->d % kCausalCg != 0)
    return fail(CAT_ERR_UNSUPPORTED, "causal CAT supports bf16 storage, N <= 256 and d a multiple of 32");
  return CAT_OK;
}

cat_status causal_mix(cat_plan plan, const float* z, const void* Vb, void* O, hipStream_t s, const LaunchTiming* t) {
  ConvArgs ca = conv_base(plan, Vb, nullptr, O);
  ca.logits = z;
  ca.ng = plan->d / kCausalCg;
  hipError_t e = launch_dconv(plan->et, ca, s, t, true);
  if (e != hipSuccess) return hip_fail(e, "causal mixing launch");
  return check_sync(plan, "causal mixing");
}

}  // namespace

extern "C" {

cat_status cat_forward_1d(cat_plan plan, const void* X, const void* W_A, const void* W_V, void* O,
                          void* workspace, void* stream) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  if (plan->p.kind != CAT_1D) return fail(CAT_ERR_PLAN_MISMATCH, "plan is not 1D");
  if (plan->p.B == 0) return CAT_OK;  // empty batch: nothing to do
  cat_status st = check_ptrs({X, W_A, W_V, O, workspace});
  if (st != CAT_OK) return st;
  return cat::forward_1d_checked(plan, X, W_A, W_V, O, workspace, stream);
}

}  // extern "C"

namespace cat {

size_t plan_forward_ws_bytes(const cat_plan_s* plan) { return plan ? plan->fwd_ws_bytes : 0; }

cat_status plan_check_forward_1d(const cat_plan_s* plan, const void* X, const void* W_A, const void* W_V,
                                 const void* O) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  if (plan->p.kind != CAT_1D) return fail(CAT_ERR_PLAN_MISMATCH, "plan is not 1D");
  if (plan->p.B == 0) return CAT_OK;
  return check_ptrs({X, W_A, W_V, O});
}

cat_status set_error(cat_status s, const char* msg) { return fail(s, msg); }

int64_t plan_batch(const cat_plan_s* plan) { return plan->p.B; }

// The 1D forward on a workspace of at least plan_forward_ws_bytes bytes,
// arguments already checked.
cat_status forward_1d_checked(cat_plan plan, const void* X, const void* W_A, const void* W_V, void* O, void* workspace,
                              void* stream) {
  cat_status st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* Vb = ws_at(workspace, plan->off_V);
  float* z = reinterpret_cast<float*>(ws_at(workspace, plan->off_z));
  KernelMark mk(plan);

  // V = X W_V (blocked for the transform) and the logits z = X W_A in one pass
  GemmArgs ga = gemm_base(plan, X);
  ga.nseg = 1;
  ga.seg[0] = seg(W_V, Vb, (int)plan->p.D, 0, OUT_BLOCKED, plan->cg);
  ga.Wz = W_A;
  ga.z = z;
  ga.nz = (int)plan->p.H;
  hipError_t e = launch_gemm(plan->et, ga, s, mk.at(0));
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  if ((st = check_sync(plan, "projection")) != CAT_OK) return st;

  return mix_from_blocked(plan, z, Vb, O, workspace, s, &mk);
}

}  // namespace cat

extern "C" {

cat_status cat_forward_avgkey_1d(cat_plan plan, const void* X, const void* W_Q, const void* W_K, const void* W_V,
                                 void* O, void* workspace, void* stream) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  if (plan->p.kind != CAT_1D) return fail(CAT_ERR_PLAN_MISMATCH, "plan is not 1D");
  if (plan->p.B == 0) return CAT_OK;
  cat_status st = check_ptrs({X, W_Q, W_K, W_V, O, workspace});
  if (st != CAT_OK) return st;
  if ((st = avgkey_supported(plan)) != CAT_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* Vb = ws_at(workspace, plan->off_V);
  float* z = reinterpret_cast<float*>(ws_at(workspace, plan->off_z));
  KernelMark mk(plan);

  // V = X W_V (blocked for the mixing), then the averaged-key logits
  GemmArgs ga = gemm_base(plan, X);
  ga.nseg = 1;
  ga.seg[0] = seg(W_V, Vb, (int)plan->p.D, 0, OUT_BLOCKED, plan->cg);
  hipError_t e = launch_gemm(plan->et, ga, s, mk.at(0));
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  if ((st = check_sync(plan, "projection")) != CAT_OK) return st;
  if ((st = avgkey_logits(plan, X, W_Q, W_K, z, workspace, s, &mk)) != CAT_OK) return st;
  return mix_from_blocked(plan, z, Vb, O, workspace, s, &mk);
}

cat_status cat_step_avgkey_logits(cat_plan plan, const void* X, const void* W_Q, const void* W_K, float* z,
                                  void* workspace, void* stream) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  if (plan->p.kind != CAT_1D) return fail(CAT_ERR_PLAN_MISMATCH, "plan is not 1D");
  if (plan->p.B == 0) return CAT_OK;
  cat_status st = check_ptrs({X, W_Q, W_K, z, workspace});
  if (st != CAT_OK) return st;
  if ((st = avgkey_supported(plan)) != CAT_OK) return st;
  return avgkey_logits(plan, X, W_Q, W_K, z, workspace, reinterpret_cast<hipStream_t>(stream), nullptr);
}

cat_status cat_forward_causal_1d(cat_plan plan, const void* X, const void* W_A, const void* W_V, void* O,
                                 void* workspace, void* stream) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  if (plan->p.kind != CAT_1D) return fail(CAT_ERR_PLAN_MISMATCH, "plan is not 1D");
  if (plan->p.B == 0) return CAT_OK;
  cat_status st = check_ptrs({X, W_A, W_V, O, workspace});
  if (st != CAT_OK) return st;
  if ((st = causal_supported(plan)) != CAT_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* Vb = ws_at(workspace, plan->off_V);
  float* z = reinterpret_cast<float*>(ws_at(workspace, plan->off_z));
  KernelMark mk(plan);
  GemmArgs ga = gemm_base(plan, X);
  ga.nseg = 1;
  ga.seg[0] = seg(W_V, Vb, (int)plan->p.D, 0, OUT_BLOCKED, kCausalCg);
  ga.Wz = W_A;
  ga.z = z;
  ga.nz = (int)plan->p.H;
  hipError_t e = launch_gemm(plan->et, ga, s, mk.at(0));
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  if ((st = check_sync(plan, "projection")) != CAT_OK) return st;
  return causal_mix(plan, z, Vb, O, s, mk.at(2));
}

cat_status cat_step_mix_causal_1d(cat_plan plan, const float* logits, const void* V, void* O, void* workspace,
                                  void* stream) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  if (plan->p.kind != CAT_1D) return fail(CAT_ERR_PLAN_MISMATCH, "plan is not 1D");
  if (plan->p.B == 0) return CAT_OK;
  cat_status st = check_ptrs({logits, V, O, workspace});
  if (st != CAT_OK) return st;
  if ((st = causal_supported(plan)) != CAT_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* Vb = ws_at(workspace, plan->off_V);
  RelayoutArgs ra{};
  ra.src = V;
  ra.dst = Vb;
  ra.src_et = plan->et;
  ra.dst_f32 = 0;
  ra.B = (int)plan->p.B;
  ra.N = (int)plan->p.N;
  ra.D = (int)plan->p.D;
  ra.H = (int)plan->p.H;
  ra.d = plan->d;
  ra.cg = kCausalCg;
  hipError_t e = launch_relayout(ra, s);
  if (e != hipSuccess) return hip_fail(e, "relayout launch");
  return causal_mix(plan, logits, Vb, O, s, nullptr);
}

cat_status cat_forward_cat_2d(cat_plan plan, const void* X, const void* W_A, const void* W_V, void* O,
                              void* workspace, void* stream) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  if (plan->p.kind != CAT_BCCB_2D) return fail(CAT_ERR_PLAN_MISMATCH, "plan is not 2D");
  if (plan->p.B == 0) return CAT_OK;
  cat_status st = check_ptrs({X, W_A, W_V, O, workspace});
  if (st != CAT_OK) return st;
  if (plan->p.H > 32)
    return fail(CAT_ERR_UNSUPPORTED, "the CAT-scored variant supports at most 32 heads (scores fused into the GEMM)");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* Vb = ws_at(workspace, plan->off_V);
  float* z = reinterpret_cast<float*>(ws_at(workspace, plan->off_z));
  KernelMark mk(plan);

  // V = X W_V (blocked for the transform) and z = X W_A in one pass
  GemmArgs ga = gemm_base(plan, X);
  ga.nseg = 1;
  ga.seg[0] = seg(W_V, Vb, (int)plan->p.D, 0, OUT_BLOCKED, plan->cg);
  ga.Wz = W_A;
  ga.z = z;
  ga.nz = (int)plan->p.H;
  hipError_t e = launch_gemm(plan->et, ga, s, mk.at(0));
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  if ((st = check_sync(plan, "projection")) != CAT_OK) return st;

  // softmax over the grid and its 2D spectrum, then the 2D convolution
  SpecArgs sa = spec_base(plan, workspace);
  sa.logits = z;
  e = launch_spectrum(plan->geom, 0, sa, s, mk.at(2));
  if (e != hipSuccess) return hip_fail(e, "spectrum launch");
  if ((st = check_sync(plan, "spectrum")) != CAT_OK) return st;
  ConvArgs ca = conv_base(plan, Vb, sa.spec, O);
  e = run_conv_1d(plan, ca, s, mk.at(3));
  if (e != hipSuccess) return hip_fail(e, "fft-conv launch");
  return check_sync(plan, "fft-conv");
}

cat_status cat_forward_bccb_2d(cat_plan plan, const void* X, const void* W_Q, const void* W_K,
                               const void* W_V, void* O, void* workspace, void* stream) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  if (plan->p.kind != CAT_BCCB_2D) return fail(CAT_ERR_PLAN_MISMATCH, "plan is not 2D");
  if (plan->p.B == 0) return CAT_OK;  // empty batch: nothing to do
  cat_status st = check_ptrs({X, W_Q, W_K, W_V, O, workspace});
  if (st != CAT_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* Vb = ws_at(workspace, plan->off_V);
  float* Qb = reinterpret_cast<float*>(ws_at(workspace, plan->off_Q));
  float* Kb = reinterpret_cast<float*>(ws_at(workspace, plan->off_K));
  float2* part = reinterpret_cast<float2*>(ws_at(workspace, plan->off_part));
  const int D = (int)plan->p.D;
  KernelMark mk(plan);

  GemmArgs ga = gemm_base(plan, X);
  ga.nseg = 3;
  ga.seg[0] = seg(W_Q, Qb, D, 1, OUT_BLOCKED, 2);
  ga.seg[1] = seg(W_K, Kb, D, 1, OUT_BLOCKED, 2);
  ga.seg[2] = seg(W_V, Vb, D, 0, OUT_BLOCKED, plan->cg);
  hipError_t e = launch_gemm(plan->et, ga, s, mk.at(0));
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  if ((st = check_sync(plan, "projection")) != CAT_OK) return st;

  ScoreArgs sc{};
  sc.Q = Qb;
  sc.K = Kb;
  sc.partial = part;
  sc.BH = (int)(plan->p.B * plan->p.H);
  sc.N = (int)plan->p.N;
  sc.npair = plan->npair;
  sc.ngrp = plan->ngrp;
  sc.ppg = plan->ppg;
  sc.et = ET_F32;
  sc.cg = 2;
  e = launch_score_partial(plan->geom, sc, s, mk.at(1));
  if (e != hipSuccess) return hip_fail(e, "score launch");
  if ((st = check_sync(plan, "scores")) != CAT_OK) return st;
  float2* psum = reinterpret_cast<float2*>(ws_at(workspace, plan->off_psum));
  e = launch_psum(part, psum, sc.BH, plan->ngrp, plan->L, s, mk.at(4));
  if (e != hipSuccess) return hip_fail(e, "partial-sum launch");
  if ((st = check_sync(plan, "partial sum")) != CAT_OK) return st;

  SpecArgs sa = spec_base(plan, workspace);
  sa.partial = psum;
  sa.ngrp = 1;
  sa.scale = 1.0f / std::sqrt((float)plan->d);
  e = launch_spectrum(plan->geom, 1, sa, s, mk.at(2));
  if (e != hipSuccess) return hip_fail(e, "spectrum launch");
  if ((st = check_sync(plan, "spectrum")) != CAT_OK) return st;

  ConvArgs ca = conv_base(plan, Vb, sa.spec, O);
  e = run_conv_1d(plan, ca, s, mk.at(3));
  if (e != hipSuccess) return hip_fail(e, "fft-conv launch");
  return check_sync(plan, "fft-conv");
}

cat_status cat_step_project(cat_plan plan, const void* X, const void* W_A, const void* W_K,
                            const void* W_V, void* V, void* z, void* K_out, void* stream) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  if (plan->p.B == 0) return CAT_OK;
  const bool two_d = plan->p.kind == CAT_BCCB_2D;
  cat_status st = two_d ? check_ptrs({X, W_A, W_K, W_V, V, z, K_out}) : check_ptrs({X, W_A, W_V, V, z});
  if (st != CAT_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int D = (int)plan->p.D;
  GemmArgs ga = gemm_base(plan, X);
  if (!two_d) {
    // the forward path's kernel: value GEMM with the fused score projection
    ga.nseg = 1;
    ga.seg[0] = seg(W_V, V, D, 0, OUT_ROWMAJOR, 1);
    ga.Wz = W_A;
    ga.z = reinterpret_cast<float*>(z);
    ga.nz = (int)plan->p.H;
  } else {
    ga.nseg = 3;
    ga.seg[0] = seg(W_A, z, D, 1, OUT_ROWMAJOR, 1);
    ga.seg[1] = seg(W_K, K_out, D, 1, OUT_ROWMAJOR, 1);
    ga.seg[2] = seg(W_V, V, D, 0, OUT_ROWMAJOR, 1);
  }
  hipError_t e = launch_gemm(plan->et, ga, s);
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  return check_sync(plan, "projection");
}

cat_status cat_step_spectrum(cat_plan plan, const float* logits, float* probs, float* spec, void* stream) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  if (plan->p.B == 0) return CAT_OK;
  cat_status st = check_ptrs({logits, spec});
  if (st != CAT_OK) return st;
  if (probs && !aligned16(probs)) return fail(CAT_ERR_INVALID_ARG, "probs not 16-byte aligned");
  if (plan->longn) return fail(CAT_ERR_UNSUPPORTED, "the spectrum step covers single-workgroup lines (the multi-pass path keeps its spectrum internal)");
  SpecArgs a{};
  a.logits = logits;
  a.probs = probs;
  a.spec = reinterpret_cast<float2*>(spec);
  a.tw = plan->d_tw;
  a.BH = (int)(plan->p.B * plan->p.H);
  a.N = (int)plan->p.N;
  a.scale = 1.0f;
  a.G = plan->Gs;
  hipError_t e = launch_spectrum(plan->geom, 0, a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "spectrum launch");
  return check_sync(plan, "spectrum");
}


cat_status cat_step_mix(cat_plan plan, const float* logits, const void* V, void* O, void* workspace,
                        void* stream) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  if (plan->p.B == 0) return CAT_OK;
  cat_status st = check_ptrs({logits, V, O, workspace});
  if (st != CAT_OK) return st;
  return mix_impl(plan, logits, V, O, workspace, reinterpret_cast<hipStream_t>(stream));
}

cat_status cat_step_mix_backward_1d(cat_plan plan, const float* logits, const void* V, const void* dO,
                                    float* dlogits, void* dV, void* workspace, void* stream) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  if (plan->p.kind != CAT_1D) return fail(CAT_ERR_PLAN_MISMATCH, "plan is not 1D");
  if (plan->p.B == 0) return CAT_OK;
  cat_status st = check_ptrs({logits, V, dO, dlogits, dV, workspace});
  if (st != CAT_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  KernelMark mk(plan);
  return mix_backward_core(plan, logits, V, dO, dlogits, dV, workspace, s, &mk);
}

cat_status cat_backward_1d(cat_plan plan, const void* X, const void* W_A, const void* W_V, const void* dO, void* dX,
                           void* dW_A, void* dW_V, void* workspace, void* stream) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  if (plan->p.kind != CAT_1D) return fail(CAT_ERR_PLAN_MISMATCH, "plan is not 1D");
  const int B = (int)plan->p.B, D = (int)plan->p.D, H = (int)plan->p.H;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  cat_status st;
  if (B == 0) {
    // an empty batch: the weight gradients are empty sums
    if ((st = check_ptrs({dW_A, dW_V})) != CAT_OK) return st;
    hipError_t e = launch_zero(dW_A, (size_t)D * H * plan->esz, s);
    if (e == hipSuccess) e = launch_zero(dW_V, (size_t)D * D * plan->esz, s);
    if (e != hipSuccess) return hip_fail(e, "zero launch");
    return check_sync(plan, "backward");
  }
  if ((st = check_ptrs({X, W_A, W_V, dO, dX, dW_A, dW_V, workspace})) != CAT_OK) return st;
  KernelMark mk(plan);
  hipError_t e;
  if ((e = hipEventRecord(plan->fork_ev, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if ((e = hipStreamWaitEvent(plan->side, plan->fork_ev, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  // From here on every exit joins the side stream back into `s`, so no
  // work of this call can still be queued on it once the caller reuses
  // the outputs or the workspace.
  st = backward_body(plan, X, W_A, W_V, dO, dX, dW_A, dW_V, workspace, s, &mk);
  const cat_status jst = join_side(plan, s);
  if (st != CAT_OK) return st;
  if (jst != CAT_OK) return jst;
  return check_sync(plan, "backward");
}

cat_status cat_step_scores_2d(cat_plan plan, const float* Q, const float* K, float* probs, void* workspace,
                              void* stream) {
  if (!plan) return fail(CAT_ERR_INVALID_ARG, "NULL plan");
  if (plan->p.kind != CAT_BCCB_2D) return fail(CAT_ERR_PLAN_MISMATCH, "plan is not 2D");
  if (plan->p.B == 0) return CAT_OK;
  cat_status st = check_ptrs({Q, K, probs, workspace});
  if (st != CAT_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* Qb = reinterpret_cast<float*>(ws_at(workspace, plan->off_Q));
  float* Kb = reinterpret_cast<float*>(ws_at(workspace, plan->off_K));
  float2* part = reinterpret_cast<float2*>(ws_at(workspace, plan->off_part));
  RelayoutArgs ra{};
  ra.src_et = ET_F32;
  ra.dst_f32 = 1;
  ra.B = (int)plan->p.B;
  ra.N = (int)plan->p.N;
  ra.D = (int)plan->p.D;
  ra.H = (int)plan->p.H;
  ra.d = plan->d;
  ra.cg = 2;
  ra.src = Q;
  ra.dst = Qb;
  hipError_t e = launch_relayout(ra, s);
  if (e != hipSuccess) return hip_fail(e, "relayout launch");
  ra.src = K;
  ra.dst = Kb;
  e = launch_relayout(ra, s);
  if (e != hipSuccess) return hip_fail(e, "relayout launch");
  ScoreArgs sc{};
  sc.Q = Qb;
  sc.K = Kb;
  sc.partial = part;
  sc.BH = (int)(plan->p.B * plan->p.H);
  sc.N = (int)plan->p.N;
  sc.npair = plan->npair;
  sc.ngrp = plan->ngrp;
  sc.ppg = plan->ppg;
  sc.et = ET_F32;
  sc.cg = 2;
  e = launch_score_partial(plan->geom, sc, s);
  if (e != hipSuccess) return hip_fail(e, "score launch");
  if ((st = check_sync(plan, "scores")) != CAT_OK) return st;
  float2* psum = reinterpret_cast<float2*>(ws_at(workspace, plan->off_psum));
  e = launch_psum(part, psum, sc.BH, plan->ngrp, plan->L, s);
  if (e != hipSuccess) return hip_fail(e, "partial-sum launch");
  if ((st = check_sync(plan, "partial sum")) != CAT_OK) return st;
  SpecArgs sa = spec_base(plan, workspace);
  sa.partial = psum;
  sa.ngrp = 1;
  sa.scale = 1.0f / std::sqrt((float)plan->d);
  sa.probs = probs;
  e = launch_spectrum(plan->geom, 1, sa, s);
  if (e != hipSuccess) return hip_fail(e, "spectrum launch");
  return check_sync(plan, "spectrum");
}

}  // extern "C"
