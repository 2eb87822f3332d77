/*
 * kfac.h - C ABI of the single-GPU K-FAC step for AMD Instinct MI355X (gfx950).
 *
 * The library computes one GPU's per-iteration K-FAC work as defined in Osawa,
 * Tsuji, Ueno, Naruse, Yokota, Matsuoka, "Large-scale distributed second-order
 * optimization using Kronecker-factored approximate curvature for deep
 * convolutional neural networks" (CVPR 2019), cited below as [OTUNYM]:
 *   - Kronecker factors A = E[a a^T] (from a layer's input activations, patch-expanded
 *     for convolutions) and G = E[g g^T] (from the gradients of the loss with respect
 *     to the layer's outputs): Section 3.2, eq. (5); E is the mini-batch mean of
 *     Section 3.1, eq. (1).
 *   - only one triangle of each symmetric factor is kept: Section 1, contributions.
 *   - the inverse of each (damped) factor: Section 3.2, eq. (6).
 *   - the preconditioned gradient G^-1 dW A^-1: Section 3.2, eq. (7).
 *   - BatchNorm's Fisher taken diagonal: Section 1, contributions, with the
 *     empirical Fisher of Section 3.1, eq. (3).
 *
 * Conventions for every entry point:
 *   - Pointers named "device" are HIP device memory on the current device, allocated
 *     and owned by the caller. Arrays of device pointers ("const void* const* act")
 *     and every other array are host memory owned by the caller. The library reads
 *     host arrays before the call returns and keeps no pointer afterwards.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the default stream) and
 *     returns without synchronising. Outputs are valid once the stream reaches them.
 *   - Scratch memory comes from the caller as `workspace` (device, 256-byte aligned)
 *     of at least the size the matching *_workspace query returns. The library calls
 *     no allocator on these paths. Two calls in flight at once on different streams
 *     must not share a workspace.
 *   - Argument, shape and size errors are detected before anything is enqueued and
 *     returned as a negative kfac_status; nothing is written then. A failed HIP launch
 *     returns KFAC_ERR_HIP. kfac_last_error() gives the text of the last error on the
 *     calling thread.
 *   - Device pointers to fp32 data must be 4-byte aligned, to fp16 data 2-byte
 *     aligned; faster paths are taken when rows are 16-byte aligned.
 *   - Only gfx950 is supported; on any other device the calls return
 *     KFAC_ERR_UNSUPPORTED.
 */
#ifndef KFAC_H_
#define KFAC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kfac_status;
#define KFAC_OK 0
#define KFAC_ERR_INVALID (-1)      /* bad pointer, shape, count or option      */
#define KFAC_ERR_UNSUPPORTED (-2)  /* not a gfx950 device, or unsupported dtype */
#define KFAC_ERR_WORKSPACE (-3)    /* workspace NULL, misaligned or too small   */
#define KFAC_ERR_HIP (-4)          /* a HIP runtime call or launch failed       */

typedef int32_t kfac_dtype;
#define KFAC_F16 0                 /* IEEE binary16 */
#define KFAC_F32 1                 /* IEEE binary32 */
#define KFAC_F64 2                 /* IEEE binary64 (accumulation of kfac_precondition_ex) */

/* One convolution or fully connected layer. Activations are NHWC [n, h, w, c_in];
 * output gradients are NHWC [n, h_out, w_out, c_out] and must satisfy
 * h_out = (h + 2 ph - kh) / sh + 1 and w_out likewise (dilation 1, zero padding).
 * A fully connected layer is h = w = h_out = w_out = kh = kw = sh = sw = 1, ph = pw = 0.
 * With bias = 1 the activation factor gets a trailing constant-1 column, so
 * d_A = c_in*kh*kw + 1; otherwise d_A = c_in*kh*kw. d_G = c_out. */
typedef struct kfac_layer {
  int32_t n, h, w, c_in;
  int32_t h_out, w_out, c_out;
  int32_t kh, kw, sh, sw, ph, pw;
  int32_t bias;
} kfac_layer;

/* One BatchNorm layer: normalised input x-hat and output gradient, both [n, hw, c]
 * (NHWC with the spatial dimensions flattened). */
typedef struct kfac_bn {
  int32_t n, hw, c;
} kfac_bn;

/* Library version: major*10000 + minor*100 + patch. */
int32_t kfac_version(void);

/* Static description of a status code (never NULL). */
const char* kfac_status_string(kfac_status status);

/* Text of the last error raised on the calling thread ("" if none). */
const char* kfac_last_error(void);

/* ---------------------------------------------------------------------------
 * kfac_factors - Kronecker factors of `count` layers ([OTUNYM] eq. (5), eq. (1)).
 *
 * For layer l with R = n*h_out*w_out patch rows:
 *   A_l = (1/R) X^T X, X[R, d_A] the patch matrix of act[l]: row (n, oh, ow) in C
 *         order, column (i*kw + j)*c_in + ci = act[n, oh*sh+i-ph, ow*sw+j-pw, ci]
 *         (0 outside the image), then the bias column of ones;
 *   G_l = (1/R) Y^T Y, Y[R, c_out] = gout[l] viewed as rows.
 * Inputs are fp16 or fp32 (`in_dtype`, for all tensors of the call); products
 * are accumulated in fp32. Each sum is formed in fp32 and multiplied once by
 * fp32(1/R).
 * Output: A_packed[l] (d_A*(d_A+1)/2 floats) and G_packed[l] (d_G*(d_G+1)/2 floats),
 * the upper triangle row by row: element (i, j), i <= j, at i*d - i*(i-1)/2 + (j-i).
 * ema_decay = 0 overwrites the outputs (their old contents are not read); otherwise
 * out = ema_decay*out + (1 - ema_decay)*batch_value (stale curvature, [OTUNYM]
 * Section 1 contributions). 0 <= ema_decay <= 1; 1 keeps the stored factors.
 * A NULL act[l] (or gout[l]) skips that factor. Results are deterministic: the same
 * inputs give bit-identical outputs. Each input tensor must span less than 2^31
 * bytes (the kernels address it with 32-bit offsets); a larger one gives
 * KFAC_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
kfac_status kfac_factors_workspace(const kfac_layer* layers, int32_t count, kfac_dtype in_dtype,
                                   size_t* bytes);
kfac_status kfac_factors(const kfac_layer* layers, int32_t count, kfac_dtype in_dtype,
                         const void* const* act, const void* const* gout,
                         float* const* A_packed, float* const* G_packed, float ema_decay,
                         void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kfac_factors_full - kfac_factors that also writes each factor's upper triangle
 * into a full matrix, the form kfac_invert reads ([OTUNYM] eq. (5) for the
 * factor, eq. (6) for the inverse that follows; Section 1 contributions: the
 * factors are symmetric, so one triangle carries them).
 *
 * A_full / G_full: NULL, or arrays of `count` device pointers (an entry may be
 * NULL) to row-major d x d fp32 matrices, caller-owned. Where given, entry (i, j),
 * i <= j, of the factor is written to full[i*d + j] with the same bits as its
 * packed entry (after the EMA blend), i.e. what kfac_pack_sym direction 2 would
 * write; the strict lower triangle is not written. Each full matrix must not
 * overlap any other buffer of the call. Arguments and errors otherwise as for
 * kfac_factors (same workspace query); a misaligned full pointer (not 4-byte
 * aligned) gives KFAC_ERR_INVALID.
 * ------------------------------------------------------------------------- */
kfac_status kfac_factors_full(const kfac_layer* layers, int32_t count, kfac_dtype in_dtype,
                              const void* const* act, const void* const* gout,
                              float* const* A_packed, float* const* G_packed,
                              float* const* A_full, float* const* G_full, float ema_decay,
                              void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kfac_pack_sym - symmetric storage conversion ([OTUNYM] Section 1: the factors
 * are symmetric, so one triangle carries all of them).
 *
 * Matrix m is n[m] x n[m]: full[m] row-major, packed[m] its upper triangle row by
 * row (n(n+1)/2 floats, same order as kfac_factors).
 * direction 0: packed <- upper triangle of full (the lower triangle is not read).
 * direction 1: full <- symmetric matrix (both triangles written from packed).
 * direction 2: upper triangle of full <- packed; the strict lower triangle of full
 *              is not written (the input kfac_invert reads, at half the writes).
 * Pure data movement: bit-exact. full and packed must not overlap.
 * ------------------------------------------------------------------------- */
kfac_status kfac_pack_sym_workspace(int32_t count, const int32_t* n, size_t* bytes);
kfac_status kfac_pack_sym(int32_t count, const int32_t* n, float* const* full,
                          float* const* packed, int32_t direction, void* workspace,
                          size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kfac_invert - damped inverses of `count` symmetric factors ([OTUNYM] eq. (6)).
 *
 * inv[m] = (F + shift[m]*I)^-1 for F = the symmetric matrix whose upper triangle is
 * read from mat[m] (n[m] x n[m], row-major fp32; the lower triangle is not read).
 * The damping shift (Tikhonov) is per matrix, e.g. sqrt(gamma) for each Kronecker
 * factor. inv[m] receives the full symmetric inverse (both triangles, exactly
 * symmetric). inv[m] may equal mat[m] (in place); otherwise they must not overlap.
 * Method: blocked Cholesky M = U^T U without pivoting whose row panels are also
 * applied to the already-inverted leading block, so the inverse is assembled in the
 * same sweep.
 * info (device, count int32) receives 0, or the 1-based column of the first pivot
 * that is not positive and finite (the LAPACK potrf convention); inv[m] is then
 * unspecified. If chol is not NULL, chol[m] (device, n x n row-major, may be NULL
 * per matrix) receives the Cholesky factor U in its upper triangle (the strict lower
 * triangle is not written).
 * ------------------------------------------------------------------------- */
kfac_status kfac_invert_workspace(int32_t count, const int32_t* n, size_t* bytes);
/* The schedule kfac_invert runs (informational, e.g. for counting the work of its
 * kernels): *block = the block size of the factorisation, *group = block steps per
 * update launch. Returns KFAC_ERR_INVALID for NULL pointers. */
kfac_status kfac_invert_schedule(int32_t* block, int32_t* group);
kfac_status kfac_invert(int32_t count, const int32_t* n, const float* const* mat,
                        float* const* inv, const float* shift, int32_t* info,
                        float* const* chol, void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kfac_invert_refine - one refinement step of damped inverses ([OTUNYM] eq. (6)):
 *   inv[m] <- X + X E,  E = I - (mat[m] + shift[m] I) X,  X = inv[m] on entry,
 * the product mat[m] X summed in fp64 from the fp32 operands and subtracted from
 * I - shift[m] X (formed in fp32) once per element, X E summed in fp32, and the
 * correction added symmetrised ((X E + (X E)^T) / 2). mat[m] is the undamped factor
 * as a full symmetric n x n row-major fp32 matrix (both triangles, e.g. kfac_pack_sym
 * direction 1), inv[m] a full symmetric n x n approximate inverse (e.g. from
 * kfac_invert); both device, caller-owned, not overlapping; inv is updated in place.
 * shift: host array of finite values. Costs two n x n x n products per matrix. Where
 * kfac_invert reported a breakdown (info != 0) for a matrix, inv[m] holds no inverse
 * and the refined result is unspecified too.
 * Errors: KFAC_ERR_INVALID for bad sizes, NULL or misaligned pointers, an inv buffer
 * that overlaps any mat or other inv buffer (mat buffers may overlap each other), and
 * non-finite shifts; KFAC_ERR_UNSUPPORTED for n > 23170 (matrices of 2^31 bytes or
 * more); KFAC_ERR_WORKSPACE for a missing or short workspace.
 * ------------------------------------------------------------------------- */
kfac_status kfac_invert_refine_workspace(int32_t count, const int32_t* n, size_t* bytes);
kfac_status kfac_invert_refine(int32_t count, const int32_t* n, const float* const* mat,
                               const float* shift, float* const* inv, void* workspace,
                               size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kfac_precondition - G^-1 dW A^-1 per layer ([OTUNYM] eq. (7)).
 *
 * Layer l: G_inv[l] is d_g[l] x d_g[l], A_inv[l] is d_a[l] x d_a[l] (full symmetric,
 * row-major fp32, as kfac_invert writes them), grad[l] is d_g x d_a row-major
 * (fp16 or fp32 per grad_dtype; with a bias column its last column is the bias
 * gradient), out[l] is d_g x d_a row-major fp32. Computed in fp32 (fp16 gradients
 * are widened exactly). out must not overlap the inputs. Every operand must span
 * less than 2^31 bytes (d_g, d_a <= 23170); larger layers give KFAC_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
kfac_status kfac_precondition_workspace(int32_t count, const int32_t* d_g, const int32_t* d_a,
                                        size_t* bytes);
kfac_status kfac_precondition(int32_t count, const int32_t* d_g, const int32_t* d_a,
                              const float* const* G_inv, const float* const* A_inv,
                              const void* const* grad, kfac_dtype grad_dtype,
                              float* const* out, void* workspace, size_t ws_bytes,
                              void* stream);

/* ---------------------------------------------------------------------------
 * kfac_precondition_update - kfac_precondition followed by the parameter update
 * of [OTUNYM] eq. (8), w <- w - lr * P with P the preconditioned gradient of
 * eq. (7), applied to each tile of P as it is formed (P is never re-read).
 *
 * w[l] (device, d_g x d_a row-major fp32, the layout of grad[l]; bias weights in
 * the last column) is updated in place. out may be NULL (P is then not stored) or
 * an array as for kfac_precondition; out[l] must not be w[l]. lr must be finite.
 * Workspace: kfac_precondition_workspace. Errors as for kfac_precondition.
 * ------------------------------------------------------------------------- */
kfac_status kfac_precondition_update(int32_t count, const int32_t* d_g, const int32_t* d_a,
                                     const float* const* G_inv, const float* const* A_inv,
                                     const void* const* grad, kfac_dtype grad_dtype,
                                     float* const* out, float* const* w, float lr,
                                     void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kfac_precondition_ex - kfac_precondition (w NULL) or kfac_precondition_update
 * (w given) with a choice of accumulation for both products ([OTUNYM] eq. (7),
 * eq. (8)): accum = KFAC_F32 as those calls, or KFAC_F64, where each product of
 * fp32 operands is formed exactly and summed in fp64 (fp64 MFMA), rounded once per
 * output element (the intermediate G^-1 dW is kept in fp32). A real weight
 * gradient lies in the range of its layer's factors; where a factor is
 * rank-deficient and the damping small, the terms of the products cancel by a large
 * factor and fp32 sums lose that many digits of the result, fp64 sums do not. The
 * fp64 MFMA rate is half the fp32 rate. Workspace: kfac_precondition_workspace.
 * Errors as for kfac_precondition; another accum gives KFAC_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
kfac_status kfac_precondition_ex(int32_t count, const int32_t* d_g, const int32_t* d_a,
                                 const float* const* G_inv, const float* const* A_inv,
                                 const void* const* grad, kfac_dtype grad_dtype,
                                 float* const* out, float* const* w, float lr, kfac_dtype accum,
                                 void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kfac_bn_diag - diagonal Fisher of BatchNorm gamma/beta ([OTUNYM] Section 1
 * contributions; diagonal of the empirical Fisher of eq. (3)).
 *
 * Layer l: xhat[l], gout[l] are [n, hw, c] (fp16 or fp32 per in_dtype). Per sample
 * s_gamma[n,c] = sum_hw gout*xhat, s_beta[n,c] = sum_hw gout (fp32 accumulation).
 * fisher[l] ([2][c] fp32: row 0 gamma, row 1 beta) <- mean_n s^2, blended as
 * fisher = ema_decay*fisher + (1-ema_decay)*batch when ema_decay != 0 (old contents
 * not read when ema_decay = 0; ema_decay = 1 keeps the stored Fisher, the stale
 * curvature case). precond[l] ([2][c] fp32) <- (mean_n s)/(fisher+shift) with the
 * blended fisher. 0 <= ema_decay <= 1.
 * ------------------------------------------------------------------------- */
kfac_status kfac_bn_diag_workspace(const kfac_bn* layers, int32_t count, size_t* bytes);
kfac_status kfac_bn_diag(const kfac_bn* layers, int32_t count, kfac_dtype in_dtype,
                         const void* const* xhat, const void* const* gout,
                         float* const* fisher, float* const* precond, float ema_decay,
                         float shift, void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kfac_bn_update - kfac_bn_diag followed by the update of [OTUNYM] eq. (8) for
 * the BatchNorm parameters: params[l] ([2][c] fp32 device: row 0 gamma, row 1
 * beta) <- params[l] - lr * precond[l], in the same kernel that forms precond.
 * params[l] must not be fisher[l] or precond[l]; lr must be finite. Workspace:
 * kfac_bn_diag_workspace. Errors as for kfac_bn_diag.
 * ------------------------------------------------------------------------- */
kfac_status kfac_bn_update(const kfac_bn* layers, int32_t count, kfac_dtype in_dtype,
                           const void* const* xhat, const void* const* gout,
                           float* const* fisher, float* const* precond, float* const* params,
                           float lr, float ema_decay, float shift, void* workspace,
                           size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kfac_bn_diag_noalloc - kfac_bn_diag (params NULL) or kfac_bn_update (params
 * given) for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. There is no
 * workspace argument and the call allocates nothing: its scratch (descriptor tables
 * and partial sums) is a static device buffer of KFAC_BN_NOALLOC_SCRATCH_BYTES per
 * GPU, part of the loaded library and held until the process ends. Layers whose
 * scratch exceeds the buffer together run in several passes; a single layer that
 * needs more than the buffer gives KFAC_ERR_INVALID (kfac_bn_diag with a workspace
 * has no such limit; at 64 channels and 112x112 positions a layer fits up to about
 * 1200 samples). Every call on a GPU shares that GPU's buffer: calls that overlap in
 * time on one GPU (other streams, other threads) race and must be ordered by the
 * caller. Results are bit-identical to kfac_bn_diag / kfac_bn_update on the same
 * inputs. Other arguments, layouts and errors as for those calls.
 * ------------------------------------------------------------------------- */
#define KFAC_BN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
kfac_status kfac_bn_diag_noalloc(const kfac_bn* layers, int32_t count, kfac_dtype in_dtype,
                                 const void* const* xhat, const void* const* gout,
                                 float* const* fisher, float* const* precond, float* const* params,
                                 float lr, float ema_decay, float shift, void* stream);

/* ---------------------------------------------------------------------------
 * Per-kernel event timing, for measurement. When enabled on a thread, every
 * kernel the library launches from that thread is bracketed by two HIP events on
 * the launch stream. kfac_timing_read synchronises those events and returns, per
 * kernel id, the summed duration in milliseconds and the number of launches since
 * the last reset. Ids run from 0 to kfac_timing_kernels()-1; kfac_kernel_name(id)
 * names them. Disabled by default; costs nothing when disabled.
 * kfac_timing_only(id) restricts the bracketing to the kernel id (events on every
 * launch cost stream time of their own), id = -1 to every kernel again (the
 * default); ids outside [-1, kfac_timing_kernels()) give KFAC_ERR_INVALID. An id
 * names one role of a kernel (the refinement's products have ids of their own).
 * ------------------------------------------------------------------------- */
int32_t kfac_timing_kernels(void);
const char* kfac_kernel_name(int32_t id);
kfac_status kfac_timing_enable(int32_t on);
kfac_status kfac_timing_only(int32_t id);
kfac_status kfac_timing_reset(void);
kfac_status kfac_timing_read(int32_t id, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* KFAC_H_ */
