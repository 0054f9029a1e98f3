/* Runs every function of the fp64 oracle (oracle/cat_oracle.c) once on small
 * inputs with odd sizes, rows subsets and ragged shapes, so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer checks its indexing.  It
 * prints nothing and returns 0 when no sanitizer fires; it does not check
 * values (tests/test_oracle.py does). */
#include <stdint.h>
#include <stdlib.h>

int oracle_num_threads(void);
void oracle_matmul(const double* X, const double* W, double* Y, int64_t M, int64_t K, int64_t Nc);
void oracle_scores_1d(const double* X, const double* WA, double* z, int64_t B, int64_t N, int64_t D, int64_t H);
void oracle_softmax_rows(const double* in, double* out, int64_t R, int64_t L);
void oracle_circulant_1d(const double* w, const double* V, double* O, int64_t B, int64_t N, int64_t D, int64_t H,
                         const int64_t* rows, int64_t nrows);
void oracle_circulant_1d_transpose(const double* w, const double* G, double* dV, int64_t B, int64_t N, int64_t D,
                                   int64_t H);
void oracle_circulant_1d_grad_w(const double* G, const double* V, double* dw, int64_t B, int64_t N, int64_t D,
                                int64_t H);
void oracle_scores_bccb_2d(const double* Q, const double* K, double* a, int64_t B, int64_t Hg, int64_t Wg, int64_t D,
                           int64_t H, double scale);
void oracle_bccb_2d(const double* w, const double* V, double* O, int64_t B, int64_t Hg, int64_t Wg, int64_t D,
                    int64_t H, const int64_t* rows, int64_t nrows);
void oracle_causal_1d(const double* z, const double* V, double* O, int64_t B, int64_t N, int64_t D, int64_t H,
                      const int64_t* rows, int64_t nrows);

static double* filled(int64_t n, unsigned seed) {
  double* p = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  for (int64_t i = 0; i < n; ++i) {
    seed = seed * 1664525u + 1013904223u;
    p[i] = (double)(seed >> 8) / 16777216.0 - 0.5;
  }
  return p;
}

int main(void) {
  if (oracle_num_threads() < 1) return 1;
  /* 1D: B = 2, N = 7 (odd), D = 6, H = 3 (d = 2) */
  const int64_t B = 2, N = 7, D = 6, H = 3;
  double* X = filled(B * N * D, 1);
  double* W = filled(D * D, 2);
  double* WA = filled(D * H, 3);
  double* Y = filled(B * N * D, 0);
  double* z = filled(B * H * N, 0);
  double* zs = filled(B * H * N, 0);
  double* O = filled(B * N * D, 0);
  double* dV = filled(B * N * D, 0);
  double* dw = filled(B * H * N, 0);
  oracle_matmul(X, W, Y, B * N, D, D);
  oracle_scores_1d(X, WA, z, B, N, D, H);
  oracle_softmax_rows(z, zs, B * H, N);
  oracle_circulant_1d(zs, Y, O, B, N, D, H, NULL, 0);
  const int64_t rows[3] = {0, 6, 13};
  oracle_circulant_1d(zs, Y, O, B, N, D, H, rows, 3);
  oracle_causal_1d(z, Y, O, B, N, D, H, NULL, 0);
  oracle_causal_1d(z, Y, O, B, N, D, H, rows, 3);
  oracle_circulant_1d_transpose(zs, X, dV, B, N, D, H);
  oracle_circulant_1d_grad_w(X, Y, dw, B, N, D, H);
  /* N = 1 */
  oracle_circulant_1d(zs, Y, O, 1, 1, D, H, NULL, 0);
  oracle_causal_1d(z, Y, O, 1, 1, D, H, NULL, 0);
  /* 2D: B = 1, 3 x 5 grid, D = 4, H = 2 */
  const int64_t Hg = 3, Wg = 5, N2 = Hg * Wg, D2 = 4, H2 = 2;
  double* Q = filled(N2 * D2, 4);
  double* K = filled(N2 * D2, 5);
  double* V2 = filled(N2 * D2, 6);
  double* a = filled(H2 * N2, 0);
  double* as = filled(H2 * N2, 0);
  double* O2 = filled(N2 * D2, 0);
  oracle_scores_bccb_2d(Q, K, a, 1, Hg, Wg, D2, H2, 0.5);
  oracle_softmax_rows(a, as, H2, N2);
  oracle_bccb_2d(as, V2, O2, 1, Hg, Wg, D2, H2, NULL, 0);
  const int64_t rows2[2] = {0, 14};
  oracle_bccb_2d(as, V2, O2, 1, Hg, Wg, D2, H2, rows2, 2);
  free(X); free(W); free(WA); free(Y); free(z); free(zs); free(O); free(dV); free(dw);
  free(Q); free(K); free(V2); free(a); free(as); free(O2);
  return 0;
}
