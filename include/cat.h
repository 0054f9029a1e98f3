/*
 * cat.h -- C ABI of the MI355X (gfx950) circulant softmax attention library
 * (libcat.so).
 *
 * What it computes
 * ----------------
 * 1D, CAT (CAT: Circular-Convolutional Attention for Sub-Quadratic
 * Transformers, "Method details / Overall framework" and "Key designs"):
 *   for every image/sequence b and head h (channels [h d, (h+1) d), d = D/H):
 *     z_h  = X_b W_A[:, h]                       (N logits, no scale, no bias)
 *     z*_h = softmax over the N tokens of z_h
 *     V    = X_b W_V
 *     O_b[:, head h] = circ(z*_h) V[:, head h],  circ(w)[i][j] = w[(i - j) mod N]
 *   evaluated as IFFT(FFT(z*_h) . FFT(V_h)) along the tokens ("Key designs:
 *   FFT-accelerated computation"), or, in bf16 for N <= 256, as the product with
 *   circ(z*_h) itself on the matrix cores (the same page notes that at
 *   N = 256 the FFT's overhead cancels its advantage; see
 *   cat_plan_conv_path).  There is no output projection.
 *
 * 2D, BCCB circulant attention (Vision Transformers are Circulant Attention
 * Learners, "What does this finding overturn?" and "Circulant Attention:
 * attention rebuilt with the FFT"), tokens in raster order n = r Wg + c on an
 * Hg x Wg grid:
 *     Q, K, V = X_b W_Q, X_b W_K, X_b W_V
 *     a_h[s]  = (1/sqrt(d)) sum_{c in head h} sum_m Q[m][c] K[(m - s) mod grid][c]
 *     a*_h    = softmax over all N = Hg Wg positions of a_h
 *     O_b[:, head h] = BCCB(a*_h) V[:, head h]      (2D circular convolution)
 *
 * Data
 * ----
 * All buffers are device memory, dense, row-major, owned by the caller:
 *   X [B][N][D], W_A [D][H], W_V / W_Q / W_K [D][D] (the products are X W as
 *   the pages write them; a torch nn.Linear weight is the transpose),
 *   O [B][N][D].
 * Storage dtype (CAT_F32 or CAT_BF16) is the same for X, the weights and O;
 * accumulation is fp32 throughout (bf16 inputs are widened exactly, O is
 * rounded to nearest even).  Two bf16 paths multiply in lower precision:
 * CAT_PATH_FFT_MATRIX runs its DFT products on fp16 operands (1D, each line
 * scaled by a power of two) or bf16 operands (2D), and CAT_PATH_DIRECT
 * rounds the softmax weights to bf16 for its products; CAT_CONV=valu (see
 * cat_plan_conv_path) keeps every product in fp32.  X, the weights, O and the workspace must be 16-byte
 * aligned; O must not overlap X, the weights or the workspace.
 *
 * Calls
 * -----
 * Forward calls only enqueue work ordered after everything already queued on
 * `stream` (a hipStream_t passed as void*; NULL is the default stream), and
 * everything queued on `stream` afterwards runs after it; every kernel of a
 * call runs on `stream` (1D: projection with the fused score projection,
 * softmax + spectrum, fft-conv).  Calls never allocate, never
 * synchronise, and return as soon as the work is queued (cat_backward_1d
 * also uses one plan-owned stream, joined back to `stream` before it
 * returns).  A plan owns small device tables (and, for 1D plans on
 * single-workgroup lines, that stream and two events) created at plan
 * creation; the workspace (size from
 * cat_plan_workspace_size) holds the intermediates and is owned by the
 * caller.  Calls that share a plan and workspace must be ordered (same stream).
 *
 * Errors
 * ------
 * Every entry returns a cat_status and never aborts.  Bad shapes, NULL
 * pointers, misalignment and a plan of the wrong kind are rejected before any
 * HIP call.  cat_last_error() returns a message for the calling thread's last
 * failure.  Setting the environment variable CAT_DEBUG_SYNC=1 makes every
 * launch synchronise and check for asynchronous errors.
 *
 * Tuning: the projection GEMM picks its output tile (128 or 256 rows by 96,
 * 128 or 192 columns) from the problem; CAT_GEMM_TILE_N=96|128|192 and
 * CAT_GEMM_TILE_M=128|256, read when a plan is created, force a width or a
 * height for that plan's calls (192 columns only where the GEMM's staged
 * 2-byte epilogue applies, 256 rows only with 2-byte operands and 128 or 192
 * columns; elsewhere the choice falls back to an allowed one).  They change
 * speed, never results beyond rounding order.
 */
#ifndef CAT_H_
#define CAT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cat_plan_s* cat_plan;

typedef enum {
  CAT_OK = 0,
  CAT_ERR_INVALID_ARG = -1,   /* bad shape, NULL pointer, misalignment */
  CAT_ERR_UNSUPPORTED = -2,   /* valid problem outside what the kernels cover */
  CAT_ERR_HIP = -3,           /* a HIP runtime call or launch failed */
  CAT_ERR_ALLOC = -4,         /* host or device allocation in plan creation failed */
  CAT_ERR_PLAN_MISMATCH = -5  /* plan built for the other kind */
} cat_status;

typedef enum { CAT_F32 = 0, CAT_BF16 = 1 } cat_dtype;
typedef enum { CAT_1D = 0, CAT_BCCB_2D = 1 } cat_kind;

/* Problem description.  1D: Hg = Wg = 0.  2D: N must equal Hg * Wg.
 * Requirements: B >= 0 (B = 0 makes every forward call a no-op), N, D,
 * H >= 1; D % H == 0; d = D / H even; D % 8 == 0; B * N * D < 2^31.
 * Supported sizes (else CAT_ERR_UNSUPPORTED):
 *   1D: H <= 32; N a power of two up to 65536, or any other N up to 32768
 *       (the circular convolution of length N is evaluated exactly on a
 *       power-of-two circle of length L >= 2N - 1, the values zero-extended
 *       and the softmaxed scores periodically extended); a power-of-two N
 *       beyond 4096, and any other N beyond 2048, by three passes over HBM
 *       (see cat_plan_conv_path);
 *   2D: grids 1x1, 2x3, 3x4, 4x4, 6x8, 8x8, 12x12, 16x16, 32x32, 96x96, and the
 *       vision-transformer patch grids 7x7, 14x14, 24x24, 28x28, 48x48. */
typedef struct {
  int32_t kind;  /* cat_kind */
  int32_t dtype; /* cat_dtype */
  int64_t B, N, D, H;
  int64_t Hg, Wg;
} cat_problem;

/* Validate `p`, choose the transform geometry and build the device tables.
 * On success *out owns host memory and device tables until cat_plan_destroy.
 * On failure *out is NULL. */
cat_status cat_plan_create(cat_plan* out, const cat_problem* p);

/* Free a plan (NULL is accepted and ignored).  No work may be in flight. */
cat_status cat_plan_destroy(cat_plan plan);

/* Bytes of device workspace every call of this plan needs (the forward
 * calls, the step calls, cat_step_mix_backward_1d and cat_forward_cat_2d
 * all fit in it). */
cat_status cat_plan_workspace_size(cat_plan plan, size_t* bytes);

/* Length of the transform circle / grid the plan uses (L, and L1 x L2 of
 * its two passes).  Diagnostic. */
cat_status cat_plan_geometry(cat_plan plan, int64_t* L, int64_t* L1, int64_t* L2);

/* How the plan evaluates the circulant mixing (diagnostic).  *path:
 *   CAT_PATH_FFT_VALU   (0) transforms on the vector ALU, with a separate
 *                           softmax-spectrum launch (2D and 1D plans that
 *                           no other path takes);
 *   CAT_PATH_FFT_MATRIX (1) 1D, L = 1024, bf16: radix-32 DFT passes on the
 *                           matrix cores, softmax spectrum computed in the
 *                           same launch; 2D, square grids of 32 or 96 a
 *                           side, bf16, d a multiple of 8: each 1D DFT pass
 *                           over the grid is one dense DFT-matrix product on
 *                           the matrix cores (bf16 operands, fp32
 *                           accumulation);
 *   CAT_PATH_DIRECT     (2) 1D, bf16, N <= 256, d a multiple of 32: the product
 *                           circ(z*_h) V_h formed directly on the matrix
 *                           cores, softmax in the same launch (CAT, "Key
 *                           designs: circulant attention matrix
 *                           construction").
 *   CAT_PATH_FFT_MULTIPASS (3) 1D, power-of-two N in (4096, 65536] or
 *                           other N in (2048, 32768]: the
 *                           transform does not fit one workgroup; column,
 *                           row and inverse column passes over HBM (CAT,
 *                           "Key designs: FFT-accelerated computation";
 *                           the page names N > 10^4 as where it should pay).
 * The environment variable CAT_CONV=fft (at plan creation) excludes path 2,
 * CAT_CONV=valu paths 1 and 2 (in 1D and 2D).  Errors: CAT_ERR_INVALID_ARG for a NULL plan
 * or NULL path. */
#define CAT_PATH_FFT_VALU 0
#define CAT_PATH_FFT_MATRIX 1
#define CAT_PATH_DIRECT 2
#define CAT_PATH_FFT_MULTIPASS 3
cat_status cat_plan_conv_path(cat_plan plan, int* path);

/* CAT 1D forward (see top of file).  X [B][N][D], W_A [D][H], W_V [D][D],
 * O [B][N][D] in the plan's storage dtype. */
cat_status cat_forward_1d(cat_plan plan, const void* X, const void* W_A, const void* W_V,
                          void* O, void* workspace, void* stream);

/* 2D BCCB circulant attention forward (see top of file).  X [B][Hg Wg][D],
 * W_Q, W_K, W_V [D][D], O [B][Hg Wg][D]. */
cat_status cat_forward_bccb_2d(cat_plan plan, const void* X, const void* W_Q, const void* W_K,
                               const void* W_V, void* O, void* workspace, void* stream);

/* CAT-scored 2D variant on a 2D plan: CAT's per-head scores on the token
 * grid as the filter of the BCCB mixing.  z_h = X W_A[:, h] (CAT:
 * Circular-Convolutional Attention for Sub-Quadratic Transformers, "Method
 * details / Overall framework"), z*_h = softmax over all Hg Wg tokens, and
 * O_h = BCCB(z*_h) V_h with V = X W_V, i.e. the 2D circular convolution
 * O[(i1, i2)] = sum_j z*[((i1 - j1) mod Hg, (i2 - j2) mod Wg)] V[j]
 * (Vision Transformers are Circulant Attention Learners, "Circulant
 * Attention: attention rebuilt with the FFT", with its filter from the
 * CAT score projection instead of the Q/K correlation).  X [B][Hg Wg][D],
 * W_A [D][H], W_V [D][D], O [B][Hg Wg][D], storage dtype, caller-owned
 * device memory.  Errors: CAT_ERR_PLAN_MISMATCH for a 1D plan;
 * CAT_ERR_UNSUPPORTED for H > 32; CAT_ERR_INVALID_ARG for NULL or
 * misaligned pointers. */
cat_status cat_forward_cat_2d(cat_plan plan, const void* X, const void* W_A, const void* W_V, void* O,
                              void* workspace, void* stream);

/* Per-kernel timing (diagnostic).  While enabled, each forward call launches
 * every kernel with a start and a stop event that the kernel's own dispatch
 * stamps (hipExtLaunchKernel), into plan-owned slots (events are created
 * here, not in the forward calls; the last 256 calls are kept, at most 32
 * launches each).  Enabling resets the slots.  cat_plan_kernel_times waits
 * for the recorded events and returns, per kernel of the path (1D:
 * projection, spectrum, fft-conv -- the mixing launch of whichever path the
 * plan takes -- then the mixing backward's own: logits reversal, relayout,
 * score-gradient partials, partial sum, logits gradient, then the
 * averaged-key logits (four launches per call); 2D: projection,
 * scores, spectrum, fft-conv, partial-score sum), the summed milliseconds
 * and the number of launches measured; *nkernels receives the number of
 * kernels (arrays hold at least 16).  cat_forward_* and
 * cat_step_mix_backward_1d record; the other step calls do not.  The
 * causal forward records its mixing launch as the fft-conv kind. */
cat_status cat_plan_set_timing(cat_plan plan, int enable);
cat_status cat_plan_kernel_times(cat_plan plan, double* total_ms, int64_t* launches, int* nkernels);

const char* cat_status_string(cat_status s);
/* Message of the calling thread's last failed call ("" if none). */
const char* cat_last_error(void);

/* ---- Step entry points: one step of the forward path each, with plain
 * row-major inputs and outputs.  For testing and diagnosis of the
 * individual steps; they share the kernels of the forward calls. */

/* Projection step.  1D plan: V [B][N][D] (storage dtype) = X W_V and
 * z [B][H][N] (fp32) = logits X W_A (W_K ignored).  2D plan: Q, K [B][N][D]
 * fp32 = X W_Q, X W_K and V (storage dtype) = X W_V; pass W_A = W_Q,
 * z = Q (fp32 [B][N][D]) and K_out for K.  No workspace is used. */
cat_status cat_step_project(cat_plan plan, const void* X, const void* W_A, const void* W_K,
                            const void* W_V, void* V, void* z, void* K_out, void* stream);

/* Softmax + filter spectrum step from logits.  logits [B][H][N] fp32 (1D: z;
 * 2D: the scaled scores a).  probs [B][H][N] fp32 receives the softmax
 * (may be NULL); spec [B][H][L] complex fp32 (interleaved re, im) receives
 * FFT_L of the (extended) softmax times 1/L in the kernels' spectral order
 * k1 + L1 k2 with natural frequency k1 + L1 k2 in 1D and (k_r = k1,
 * k_c = k2) on a 2D grid.  Plans on CAT_PATH_FFT_MULTIPASS return
 * CAT_ERR_UNSUPPORTED (their spectrum lives only inside cat_step_mix). */
cat_status cat_step_spectrum(cat_plan plan, const float* logits, float* probs, float* spec,
                             void* stream);

/* Circulant mixing step: O = circ(softmax(logits)) V per head (1D) or
 * BCCB(softmax(logits)) V (2D).  logits [B][H][N] fp32 (2D: already scaled),
 * V and O [B][N][D] storage dtype. */
cat_status cat_step_mix(cat_plan plan, const float* logits, const void* V, void* O,
                        void* workspace, void* stream);

/* Backward of the 1D mixing step (CAT is trained end to end: CAT:
 * Circular-Convolutional Attention for Sub-Quadratic Transformers, "Method
 * details / Overall framework"; the gradients are the chain rule of
 * O_h = circ(z*_h) V_h, z*_h = softmax(logits_h)).  Given the output
 * gradient dO:
 *   dV[b][j][c]      = sum_i z*[b][h][(i - j) mod N] dO[b][i][c]
 *                      (circ(z*_h)^T dO_h, evaluated as the forward mixing
 *                      of the reversed logits, on the plan's mixing path);
 *   dz*[b][h][k]     = sum over the head's channels c and tokens i of
 *                      dO[b][i][c] V[b][(i - k) mod N][c]
 *                      (a cross-correlation, by FFT on the plan's circle;
 *                      on CAT_PATH_FFT_MULTIPASS the cross-spectra of a
 *                      head's channel pairs are summed before one
 *                      three-pass inverse transform, and lags that wrap
 *                      mod N are folded back on a padded circle);
 *   dlogits[b][h][k] = z*[k] (dz*[k] - sum_m z*[m] dz*[m]).
 * logits [B][H][N] fp32 (the forward's z), V and dO [B][N][D] storage
 * dtype (all caller-owned device memory, read only); dlogits [B][H][N] fp32
 * and dV [B][N][D] storage dtype are written.  dV in bf16 is rounded from
 * fp32; dlogits is computed in fp32 from the stored V and dO.  workspace:
 * cat_plan_workspace_size bytes.  Every 1D length of the forward is
 * supported.  Errors: CAT_ERR_PLAN_MISMATCH for a 2D plan;
 * CAT_ERR_INVALID_ARG for NULL or misaligned pointers. */
cat_status cat_step_mix_backward_1d(cat_plan plan, const float* logits, const void* V, const void* dO,
                                    float* dlogits, void* dV, void* workspace, void* stream);

/* Gradients of the 1D CAT forward (cat_forward_1d) for an output gradient
 * dO [B][N][D]: dX [B][N][D], dW_A [D][H], dW_V [D][D], all in the storage
 * dtype, caller-owned device memory.  The chain rule through V = X W_V,
 * z_h = X W_A[:, h] (CAT: Circular-Convolutional Attention for
 * Sub-Quadratic Transformers, "Method details / Overall framework") and the
 * mixing (cat_step_mix_backward_1d):
 *   dW_V = X^T dV,  dW_A = X^T dz^T,  dX = dV W_V^T + dz^T W_A^T,
 * with V and z recomputed from X.  The products run on the projection
 * GEMM (fp32 accumulation; dX is accumulated in fp32 and rounded once; dV
 * and dz enter the weight products rounded to the storage dtype).
 * Every 1D length and batch of the forward is supported (X^T is staged with
 * its B N columns padded with zeros to a multiple of 8); B = 0 writes zero
 * weight gradients (dX is empty; X, W_A, W_V, dO, dX and workspace are not
 * read and may be NULL).  Errors: CAT_ERR_PLAN_MISMATCH for a 2D plan;
 * CAT_ERR_INVALID_ARG for NULL or misaligned pointers.  Streams: the
 * weight-gradient branch runs on a stream the plan owns (default priority),
 * forked from `stream` by an event after the mixing backward and joined
 * back before the call returns (on every return after the fork, errors
 * included), so every output is ordered on `stream` like any other call's.
 * Calls sharing a plan must be ordered, and two host threads must not run
 * this entry on one plan at the same time: the fork and join events belong
 * to the plan. */
cat_status cat_backward_1d(cat_plan plan, const void* X, const void* W_A, const void* W_V, const void* dO, void* dX,
                           void* dW_A, void* dW_V, void* workspace, void* stream);

/* Averaged-key variant of CAT on a 1D plan (CAT: Circular-Convolutional
 * Attention for Sub-Quadratic Transformers, ablation table, row "qkv
 * (Averaged-Key)": 3 D^2 parameters at O(N log N)).  Read as the key
 * averaged over the tokens and met by each query as in scaled dot-product
 * attention:
 *   Q = X_b W_Q,  K = X_b W_K,  kbar_h = (1/N) sum_n K_h[n],
 *   z_h[n] = Q_h[n] . kbar_h / sqrt(d),  z*_h = softmax over n,
 *   O_b[:, head h] = circ(z*_h) V[:, head h],  V = X_b W_V,
 * with the circulant mixing of cat_forward_1d on the plan's path.  The
 * logits are evaluated as X_b (W_Q,h kbar_h) / sqrt(d) with kbar =
 * (token mean of X_b) W_K -- the same sums in another association, in fp32
 * -- so Q and K are never formed.  X [B][N][D], W_Q, W_K, W_V [D][D], O
 * [B][N][D], storage dtype, caller-owned device memory.  Errors:
 * CAT_ERR_PLAN_MISMATCH for a 2D plan; CAT_ERR_UNSUPPORTED for D > 3072 or
 * B > 65535; CAT_ERR_INVALID_ARG for NULL or misaligned pointers. */
cat_status cat_forward_avgkey_1d(cat_plan plan, const void* X, const void* W_Q, const void* W_K, const void* W_V,
                                 void* O, void* workspace, void* stream);

/* The averaged-key logits alone: z [B][H][N] fp32 (caller-owned device
 * memory), as in cat_forward_avgkey_1d.  Same errors. */
cat_status cat_step_avgkey_logits(cat_plan plan, const void* X, const void* W_Q, const void* W_K, float* z,
                                  void* workspace, void* stream);

/* Causal CAT on a 1D plan (CAT: Circular-Convolutional Attention for
 * Sub-Quadratic Transformers, "Loss function / training strategy": a causal
 * language model must shift Z to stay causal, at O(N^2) cost; "Limitations
 * and outlook").  Read as standard causal masking of the circulant score
 * matrix before its row softmax: row i of circ(z_h) keeps the tokens
 * j <= i,
 *   O_b[i][c] = sum_{j <= i} exp(z_h[i - j]) V[j][c] / sum_{k <= i} exp(z_h[k]),
 * with z_h = X_b W_A[:, h] and V = X_b W_V as in cat_forward_1d, evaluated
 * as the O(N^2) direct product on the matrix cores.  The exponentials are
 * taken against the maximum of the whole line, so a row whose kept logits
 * all lie more than about 87 below it would underflow.  X [B][N][D], W_A
 * [D][H], W_V [D][D], O [B][N][D], caller-owned device memory.  Errors:
 * CAT_ERR_PLAN_MISMATCH for a 2D plan; CAT_ERR_UNSUPPORTED unless the
 * storage is bf16, N <= 256 and d is a multiple of 32; CAT_ERR_INVALID_ARG
 * for NULL or misaligned pointers. */
cat_status cat_forward_causal_1d(cat_plan plan, const void* X, const void* W_A, const void* W_V, void* O,
                                 void* workspace, void* stream);

/* The causal mixing alone: O = causal CAT mixing of V [B][N][D] (storage
 * dtype) with the logits [B][H][N] fp32, as in cat_forward_causal_1d.  Same
 * errors. */
cat_status cat_step_mix_causal_1d(cat_plan plan, const float* logits, const void* V, void* O, void* workspace,
                                  void* stream);

/* For callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid hipMalloc): the 1D
 * forward of cat_forward_1d, with the same arguments minus the workspace.
 * Its intermediates live in a fixed array of CAT_NOALLOC_SCRATCH_BYTES that
 * the library keeps in every GPU's memory from load until the process
 * ends; this call allocates and frees nothing.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race, so order them.  Nothing in the array needs clearing
 * (each call writes what it reads).  Errors: those of cat_forward_1d;
 * CAT_ERR_UNSUPPORTED when the problem needs more than
 * CAT_NOALLOC_SCRATCH_BYTES of intermediates (cat_plan_workspace_size
 * bounds it; the 1D forward needs about B N D s + 8 B H L + 4 B H N
 * bytes, s the storage bytes, more on the long path). */
#define CAT_NOALLOC_SCRATCH_BYTES (64u << 20)
cat_status cat_forward_1d_noalloc(cat_plan plan, const void* X, const void* W_A, const void* W_V, void* O,
                                  void* stream);

/* 2D score step: probs [B][H][N] fp32 = softmax over the grid of the scaled
 * circular cross-correlation of Q and K (both [B][N][D] fp32).  2D plans only. */
cat_status cat_step_scores_2d(cat_plan plan, const float* Q, const float* K, float* probs,
                              void* workspace, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CAT_H_ */
