"""Plain fp64 CPU oracle of the single-GPU K-FAC step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
module: only the test suite, the smoke check in ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` use it. It shares no code with the HIP library.

Every function is the plain definition, computed in fp64 from the exact values of
its (fp16 or fp32) inputs, written for a reader to check by eye. Library primitives
(a matrix product, a matrix-vector product) serve as single steps; nothing is blocked,
fused or reordered.

Source: Osawa, Tsuji, Ueno, Naruse, Yokota, Matsuoka, "Large-scale distributed
second-order optimization using Kronecker-factored approximate curvature for deep
convolutional neural networks" (CVPR 2019), cited as [OTUNYM]:

* Section 3.1, eq. (1): E[.] is the mean over the samples of a mini-batch.
* Section 3.1, eq. (3): the empirical Fisher is the mean outer product of per-sample
  log-likelihood gradients.
* Section 3.2, eq. (4)-(5): the Fisher is taken block-diagonal over layers and each
  block is the Kronecker product G_l (x) A_{l-1}; G comes from the loss gradients with
  respect to the layer's outputs, A from the layer's inputs.
* Section 3.2, eq. (6): the inverse of the Kronecker product is the Kronecker product
  of the inverses.
* Section 3.2, eq. (7): the preconditioned gradient is that inverse applied to the
  layer's gradient, G^-1 . dW . A^-1 in matrix form.
* Section 3.2, eq. (8): the parameters move against the preconditioned gradient,
  scaled by the learning rate.
* Section 1, list of contributions: the factors are symmetric (one triangle suffices),
  BatchNorm's Fisher is taken diagonal, and the Fisher is refreshed less often.

Readings where the pages are silent (stated again at each function):
im2col column order (kh, kw, c_in) with c_in fastest, a trailing constant-1 bias
column, E over all N*H_out*W_out patch rows, Tikhonov damping as F + s*I, an
exponential moving average for refreshed factors, and the BN Fisher as the diagonal
of eq. (3) over per-sample gradients of gamma and beta.

Pin status: every public function is pinned by ``tests/test_oracle_pins.py`` against
closed forms, exact rational brute force, library special cases or invariants. No
function here is "parity unpinned".
"""
import numpy as np

__all__ = [
    "im2col_nhwc", "gram", "second_moment", "conv_factors", "ema_update",
    "packed_offset", "pack_upper", "unpack_upper", "cholesky_upper",
    "upper_triangular_inverse", "damped_inverse", "precondition", "bn_diag_fisher",
    "sgd_update",
]


# ---------------------------------------------------------------------------
# Factors: [OTUNYM] Section 3.2, eq. (5)
# ---------------------------------------------------------------------------

def im2col_nhwc(x, kh, kw, sh, sw, ph, pw, bias):
    """Patch matrix X[R, d] of an NHWC activation tensor, in fp64.

    Row r enumerates (n, oh, ow) in C order, R = N*H_out*W_out. Column
    c = (i*kw + j)*C_in + ci holds x[n, oh*sh + i - ph, ow*sw + j - pw, ci] for tap
    (i, j) and channel ci, and 0 where that position is outside the image (zero
    padding, dilation 1). With ``bias`` one more column of ones is appended.
    Reading: the pages name A as coming from the layer's input activations but do
    not print the convolution form; this is the standard patch expansion with the
    channel index fastest, which matches NHWC storage.
    """
    x = np.asarray(x, dtype=np.float64)
    n, h, w, c = x.shape
    h_out = (h + 2 * ph - kh) // sh + 1
    w_out = (w + 2 * pw - kw) // sw + 1
    cols = np.zeros((n, h_out, w_out, kh, kw, c), dtype=np.float64)
    for i in range(kh):
        ih = np.arange(h_out) * sh + i - ph
        oh_ok = np.nonzero((ih >= 0) & (ih < h))[0]
        for j in range(kw):
            iw = np.arange(w_out) * sw + j - pw
            ow_ok = np.nonzero((iw >= 0) & (iw < w))[0]
            cols[:, oh_ok[:, None], ow_ok[None, :], i, j, :] = \
                x[:, ih[oh_ok][:, None], iw[ow_ok][None, :], :]
    X = cols.reshape(n * h_out * w_out, kh * kw * c)
    if bias:
        X = np.concatenate([X, np.ones((X.shape[0], 1))], axis=1)
    return X


def gram(X):
    """Unscaled Gram matrix X^T X in fp64 (the sum over rows of x x^T)."""
    X = np.asarray(X, dtype=np.float64)
    return X.T @ X


def second_moment(X):
    """E[x x^T] over the rows of X: X^T X / R.

    [OTUNYM] eq. (1) makes E the mean over samples; for a convolution the rows are the
    R = N*H_out*W_out patch rows (reading: one mean over all patch rows, for both A and
    G). The moment is uncentred: no mean is subtracted.
    """
    X = np.asarray(X, dtype=np.float64)
    return gram(X) / X.shape[0]


def conv_factors(act, gout, kh, kw, sh, sw, ph, pw, bias):
    """Kronecker factors of one convolution or fully connected layer.

    A = E[a a^T] over the im2col rows of the NHWC input ``act`` (with bias column),
    G = E[g g^T] over the rows of the NHWC output gradient ``gout`` reshaped to
    [R, C_out]. [OTUNYM] eq. (5): F_l ~ G_l (x) A_{l-1}. A fully connected layer is
    the case kh = kw = 1, H = W = 1.
    """
    X = im2col_nhwc(act, kh, kw, sh, sw, ph, pw, bias)
    gout = np.asarray(gout, dtype=np.float64)
    Gam = gout.reshape(-1, gout.shape[-1])
    if Gam.shape[0] != X.shape[0]:
        raise ValueError("activation patches and output gradients disagree on R")
    return second_moment(X), second_moment(Gam)


def ema_update(old, batch, decay):
    """Refreshed factor under stale curvature.

    [OTUNYM] Section 1 (contributions) reduces how often the Fisher is updated; the
    form is a reading: S <- decay*S + (1 - decay)*S_batch, and decay = 0 means the batch
    value overwrites S (the first refresh).
    """
    batch = np.asarray(batch, dtype=np.float64)
    if decay == 0.0:
        return batch.copy()
    return decay * np.asarray(old, dtype=np.float64) + (1.0 - decay) * batch


# ---------------------------------------------------------------------------
# Symmetric storage: [OTUNYM] Section 1 (the factors' symmetry halves the data)
# ---------------------------------------------------------------------------

def packed_offset(i, j, n):
    """Offset of element (i, j), i <= j, of an n x n symmetric matrix stored as its
    upper triangle row by row: rows 0..i-1 hold n, n-1, ..., n-i+1 entries."""
    if not (0 <= i <= j < n):
        raise IndexError("packed_offset needs 0 <= i <= j < n")
    return i * n - (i * (i - 1)) // 2 + (j - i)


def pack_upper(M):
    """Upper triangle of M, row by row (n(n+1)/2 entries). The lower triangle is not
    read."""
    M = np.asarray(M)
    n = M.shape[0]
    out = np.empty(n * (n + 1) // 2, dtype=M.dtype)
    for i in range(n):
        o = packed_offset(i, i, n)
        out[o:o + n - i] = M[i, i:]
    return out


def unpack_upper(p, n):
    """Full symmetric n x n matrix from its packed upper triangle (both triangles
    written; element (j, i) is a copy of element (i, j))."""
    p = np.asarray(p)
    if p.shape[0] != n * (n + 1) // 2:
        raise ValueError("packed length must be n(n+1)/2")
    M = np.empty((n, n), dtype=p.dtype)
    for i in range(n):
        o = packed_offset(i, i, n)
        M[i, i:] = p[o:o + n - i]
        M[i:, i] = p[o:o + n - i]
    return M


# ---------------------------------------------------------------------------
# Damped inverse: [OTUNYM] eq. (6)
# ---------------------------------------------------------------------------

def cholesky_upper(M):
    """M = U^T U with U upper triangular and a positive diagonal, in fp64.

    Row form of the textbook factorisation: row k of U is row k of M minus the
    contributions of rows 0..k-1 of U, divided by the square root of its diagonal
    entry (the pivot). Only the upper triangle of M is read. Returns (U, info): info is
    0, or the 1-based index of the first pivot that is not positive and finite (the
    LAPACK potrf convention), in which case rows k.. of U are left zero. No pivoting.
    """
    M = np.asarray(M, dtype=np.float64)
    n = M.shape[0]
    U = np.zeros((n, n), dtype=np.float64)
    for k in range(n):
        row = M[k, k:] - U[:k, k] @ U[:k, k:] if k else M[k, k:].copy()
        d = row[0]
        if not (np.isfinite(d) and d > 0.0):
            return U, k + 1
        U[k, k:] = row / np.sqrt(d)
    return U, 0


def upper_triangular_inverse(U):
    """X = U^-1 for upper triangular U by back substitution: row i of X follows from
    U[i, i] X[i, j] + sum_{k > i} U[i, k] X[k, j] = delta_ij, rows taken bottom-up."""
    U = np.asarray(U, dtype=np.float64)
    n = U.shape[0]
    X = np.zeros((n, n), dtype=np.float64)
    for i in range(n - 1, -1, -1):
        X[i, i] = 1.0 / U[i, i]
        if i + 1 < n:
            X[i, i + 1:] = -(U[i, i + 1:] @ X[i + 1:, i + 1:]) / U[i, i]
    return X


def damped_inverse(F, shift):
    """(F + shift*I)^-1 for a symmetric factor F, in fp64, with its breakdown index.

    [OTUNYM] eq. (6) inverts each Kronecker factor on its own. Damping is a reading
    (the pages' damping section is not on them): Tikhonov damping adds ``shift`` to the
    diagonal of each factor (shift = sqrt(gamma) per factor, so the Kronecker product
    carries about gamma). The inverse goes through the Cholesky factor:
    M = U^T U, M^-1 = U^-1 U^-T, and the result is made exactly symmetric by copying
    its upper triangle to the lower one. Only the upper triangle of F is read.
    Returns (M^-1, 0), or (None, info) when pivot ``info`` (1-based) breaks down.
    """
    F = np.asarray(F, dtype=np.float64)
    n = F.shape[0]
    M = np.triu(F) + np.triu(F, 1).T + np.float64(shift) * np.eye(n)
    U, info = cholesky_upper(M)
    if info:
        return None, info
    Ui = upper_triangular_inverse(U)
    X = Ui @ Ui.T
    X = np.triu(X) + np.triu(X, 1).T
    return X, 0


# ---------------------------------------------------------------------------
# Preconditioning: [OTUNYM] eq. (7)
# ---------------------------------------------------------------------------

def precondition(G_inv, grad, A_inv):
    """Preconditioned gradient G^-1 . dW . A^-1 of one layer, in fp64.

    [OTUNYM] eq. (6)-(7): (G (x) A)^-1 vec(dW) with dW of shape [d_G, d_A] and
    row-major vec equals vec(G^-1 dW A^-1) (A and G symmetric). The last column of dW
    is the bias gradient when A carries the bias column.
    """
    return (np.asarray(G_inv, dtype=np.float64) @ np.asarray(grad, dtype=np.float64)
            @ np.asarray(A_inv, dtype=np.float64))


# ---------------------------------------------------------------------------
# BatchNorm diagonal Fisher: [OTUNYM] Section 1 (contributions) and eq. (3)
# ---------------------------------------------------------------------------

def bn_diag_fisher(xhat, gout, shift, ema_decay=0.0, fisher_prev=None):
    """Diagonal-Fisher preconditioning of one BatchNorm layer's gamma and beta.

    ``xhat`` (normalised input) and ``gout`` (gradient of the loss with respect to the
    layer's output) are [N, HW, C]. Per sample n and channel c the gradients are
    s_gamma[n, c] = sum_hw gout * xhat and s_beta[n, c] = sum_hw gout. Reading of the
    pages' diagonal approximation: the Fisher is the diagonal of eq. (3) over these
    per-sample gradients, F[c] = mean_n s[n, c]^2, the mini-batch gradient is
    grad[c] = mean_n s[n, c], and the preconditioned gradient is grad / (F + shift).
    Under stale curvature F is blended like the Kronecker factors (see ``ema_update``).
    Returns dict(fisher=[2, C], grad=[2, C], precond=[2, C]), row 0 gamma, row 1 beta.
    """
    x = np.asarray(xhat, dtype=np.float64)
    g = np.asarray(gout, dtype=np.float64)
    s_gamma = (g * x).sum(axis=1)          # [N, C]
    s_beta = g.sum(axis=1)                 # [N, C]
    s = np.stack([s_gamma, s_beta])        # [2, N, C]
    fisher = (s * s).mean(axis=1)
    grad = s.mean(axis=1)
    if ema_decay != 0.0:
        fisher = ema_update(fisher_prev, fisher, ema_decay)
    return {"fisher": fisher, "grad": grad, "precond": grad / (fisher + np.float64(shift))}


# ---------------------------------------------------------------------------
# Parameter update: [OTUNYM] eq. (8)
# ---------------------------------------------------------------------------

def sgd_update(w, precond_grad, lr):
    """New parameters w - lr * G, in fp64.

    [OTUNYM] eq. (8): each layer's parameters take a step of size lr (the learning
    rate eta) against its preconditioned gradient G of eq. (7) (``precondition``;
    for BatchNorm gamma and beta the ``precond`` of ``bn_diag_fisher``). The pages
    give the plain step: no momentum or weight decay is applied here.
    """
    return np.asarray(w, dtype=np.float64) - np.float64(lr) * np.asarray(precond_grad, dtype=np.float64)

