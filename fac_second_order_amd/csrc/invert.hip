// Batched damped inverses (F + s I)^-1 of symmetric positive definite factors.
// Osawa et al. (CVPR 2019), Section 3.2, eq. (6): the inverse of the Kronecker
// product is the Kronecker product of the factors' inverses, so each factor is
// inverted on its own; damping adds s to the diagonal of each factor.
//
// Method: a blocked right-looking Cholesky factorisation M = U^T U (block 128, no
// pivoting) in which every block step is also applied to the rows and columns
// that were already eliminated, so the inverse is assembled in the same sweep
// (the symmetric Gauss-Jordan form of the Cholesky inverse). With S the working
// matrix (upper triangle only) and k the pivot block, one step is
//   pivot:  U_kk = chol(S_kk) and E = U_kk^-T, in one workgroup with the 128x128
//           block held in registers (one LDS row broadcast and one barrier per
//           column); also P^-1 = E^T E;
//   panel:  for every column block j != k: V_j = S_kj, Y_j = E V_j (the Cholesky
//           row panel U_kj when j > k) and W_j = E^T Y_j = P^-1 V_j, on MFMA;
//   update: S_ij -= Y_i^T Y_j for all upper tiles i, j != k (fp32 MFMA), and
//           S_kj = W_j, S_ik = W_i^T, S_kk = -P^-1.
// After the last step S = -M^-1; the finish kernel negates it and writes both
// triangles. All matrices of a call step together: they are ordered by block
// count, so the ones still active at step k are a prefix of the list.
#include <algorithm>

#include "tile_f32.hpp"

namespace kfac {

struct InvDesc {
  const float* mat;
  float* S;        // working matrix = the output buffer
  float* chol;     // optional U output (nullptr)
  int32_t* info;   // this matrix's info entry
  float* E;        // [TB][TB]  U_kk^-T (lower triangular)
  float* Ui;       // [TB][TB]  U_kk^-1 (upper triangular)
  float* Pn;       // [TB][TB]  -P^-1
  float* Y;        // [TB][n]   Y panels (rows = pivot rows)
  float* W;        // [TB][n]   W panels
  int32_t n, nb;
  float shift;
  int32_t nb64;    // 64-wide blocks (prep/finish tiles)
};

constexpr int FT = 64;  // prep/finish tile edge

// S <- upper(mat) + shift*I (S may equal mat); info <- 0.
__global__ void __launch_bounds__(256) inv_prep_kernel(const InvDesc* __restrict__ desc,
                                                       const int32_t* __restrict__ begin, int count) {
  const int p = find_problem(begin, count, blockIdx.x);
  const InvDesc& d = desc[p];
  int ti, tj;
  upper_tile(blockIdx.x - begin[p], d.nb64, ti, tj);
  const int64_t n = d.n;
  const int c = threadIdx.x & (FT - 1);
  const int64_t j = int64_t(tj) * FT + c;
  for (int r = threadIdx.x >> 6; r < FT; r += 4) {
    const int64_t i = int64_t(ti) * FT + r;
    if (i < n && j < n && i <= j) {
      float v = d.mat[i * n + j];
      if (i == j) v += d.shift;
      d.S[i * n + j] = v;
    }
  }
  if (ti == 0 && tj == 0 && threadIdx.x == 0) *d.info = 0;
}

// Pivot block of step k: Cholesky in registers, E = U^-T, P^-1 = E^T E.
// 1024 threads; thread t owns the 4x4 sub-block (rows 4*(t/32).., cols 4*(t%32)..).
__global__ void __launch_bounds__(1024) inv_pivot_kernel(const InvDesc* __restrict__ desc, int k) {
  const InvDesc& d = desc[blockIdx.x];
  const int n = d.n, k0 = k * TB, bk = min(TB, n - k0);
  const int t = threadIdx.x, br = t >> 5, bc = t & 31;
  __shared__ float zrow[2][TB], erow[2][TB];
  __shared__ float Es[TB][LDT];

  float Z[4][4], E[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = 4 * br + r, j = 4 * bc + c;
      float z = (i == j) ? 1.f : 0.f;
      if (i < bk && j < bk) {
        const int a = min(i, j), b = max(i, j);
        z = d.S[int64_t(k0 + a) * n + k0 + b];
      }
      Z[r][c] = z;
      E[r][c] = (i == j) ? 1.f : 0.f;
    }

  int failed = 0;  // 1-based local column of the first bad pivot
  for (int kk = 0; kk < bk; ++kk) {
    const int buf = kk & 1;
    if (br == (kk >> 2)) {
      const int r = kk & 3;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        zrow[buf][4 * bc + c] = Z[r][c];
        erow[buf][4 * bc + c] = E[r][c];
      }
    }
    __syncthreads();
    const float piv = zrow[buf][kk];
    if (!(piv > 0.f) || !isfinite(piv)) {  // same value in every thread: uniform exit
      failed = kk + 1;
      break;
    }
    const float sq = sqrtf(piv);
    const float rs = 1.0f / sq;
    float ui[4], uj[4], ej[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ui[q] = zrow[buf][4 * br + q] * rs;
      uj[q] = zrow[buf][4 * bc + q] * rs;
      ej[q] = erow[buf][4 * bc + q] * rs;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * br + r;
      if (i == kk) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = 4 * bc + c;
          if (j > kk) Z[r][c] = uj[c];
          else if (j == kk) Z[r][c] = sq;
          E[r][c] = ej[c];
        }
      } else if (i > kk) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = 4 * bc + c;
          if (j > kk) Z[r][c] = fmaf(-ui[r], uj[c], Z[r][c]);
          E[r][c] = fmaf(-ui[r], ej[c], E[r][c]);
        }
      }
    }
  }

#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = 4 * br + r, j = 4 * bc + c;
      Es[i][j] = E[r][c];
      d.E[i * TB + j] = E[r][c];
      d.Ui[j * TB + i] = E[r][c];
      if (d.chol && i <= j && j < bk) d.chol[int64_t(k0 + i) * n + k0 + j] = Z[r][c];
    }
  __syncthreads();
  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
  for (int q = 0; q < bk; ++q) {
    float ei[4], ej[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ei[r] = Es[q][4 * br + r];
      ej[r] = Es[q][4 * bc + r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(ei[r], ej[c], acc[r][c]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) d.Pn[(4 * br + r) * TB + 4 * bc + c] = -acc[r][c];
  if (failed && t == 0 && *d.info == 0) *d.info = k0 + failed;
}

// Panel of step k: for column block j != k, Y_j = E V_j and W_j = E^T Y_j.
__global__ void __launch_bounds__(256) inv_panel_kernel(const InvDesc* __restrict__ desc,
                                                        const int32_t* __restrict__ begin,
                                                        int count, int k) {
  const int p = find_problem(begin, count, blockIdx.x);
  const InvDesc& d = desc[p];
  const int c = blockIdx.x - begin[p];
  const int j = c < k ? c : c + 1;
  const int n = d.n, k0 = k * TB, bk = min(TB, n - k0);
  const int j0 = j * TB, bj = min(TB, n - j0);
  __shared__ float Ys[TB * LDT];
  __shared__ float As[KT * LDT], Bs[KT * LDT];

  Quad q;
  quad_zero(q);
  for (int kc = 0; kc < bk; kc += KT) {
    stage_rows(As, d.Ui, TB, kc, bk, 0, bk);            // A[p][m] = Ui[p][m] = E[m][p]
    if (j > k) stage_rows(Bs, d.S + int64_t(k0) * n + j0, n, kc, bk, 0, bj);   // V = S_kj
    else stage_cols(Bs, d.S + int64_t(j0) * n + k0, n, kc, bk, 0, bj);        // V = S_jk^T
    __syncthreads();
    quad_mma(q, As, Bs, 1.f);
    __syncthreads();
  }
  quad_to_lds(q, Ys);  // rows >= bk are zero (their A columns were zero)
  quad_store(q, d.Y + j0, n, bk, bj);
  if (d.chol && j > k) quad_store(q, d.chol + int64_t(k0) * n + j0, n, bk, bj);
  quad_zero(q);
  __syncthreads();
  for (int kc = 0; kc < bk; kc += KT) {
    stage_rows(As, d.E, TB, kc, bk, 0, bk);             // A[p][m] = E[p][m] = Ui[m][p]
    __syncthreads();
    quad_mma(q, As, Ys + kc * LDT, 1.f);
    __syncthreads();
  }
  quad_store(q, d.W + j0, n, bk, bj);
}

// Update of step k over the upper 128-tiles of every active matrix.
__global__ void __launch_bounds__(256) inv_update_kernel(const InvDesc* __restrict__ desc,
                                                         const int32_t* __restrict__ begin,
                                                         int count, int k) {
  const int p = find_problem(begin, count, blockIdx.x);
  const InvDesc& d = desc[p];
  int ti, tj;
  upper_tile(blockIdx.x - begin[p], d.nb, ti, tj);
  const int n = d.n, k0 = k * TB, bk = min(TB, n - k0);
  const int i0 = ti * TB, j0 = tj * TB;
  const int bi = min(TB, n - i0), bj = min(TB, n - j0);
  __shared__ float buf[TB * LDT];
  float* S = d.S;

  if (ti == k && tj == k) {  // S_kk = -P^-1
    for (int e = threadIdx.x; e < bk * bk; e += 256) {
      const int r = e / bk, c = e % bk;
      if (r <= c) S[int64_t(k0 + r) * n + k0 + c] = d.Pn[r * TB + c];
    }
    return;
  }
  if (ti == k) {  // S_kj = W_j (rows of the pivot block)
    for (int e = threadIdx.x; e < bk * bj; e += 256) {
      const int r = e / bj, c = e % bj;
      S[int64_t(k0 + r) * n + j0 + c] = d.W[int64_t(r) * n + j0 + c];
    }
    return;
  }
  if (tj == k) {  // S_ik = W_i^T (column of the pivot block, above it)
    for (int e = threadIdx.x; e < bk * bi; e += 256) {
      const int r = e / bi, c = e % bi;  // W row r (pivot row), column i0 + c
      buf[r * LDT + c] = d.W[int64_t(r) * n + i0 + c];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < bi * bk; e += 256) {
      const int r = e / bk, c = e % bk;  // S row i0 + r, column k0 + c
      S[int64_t(i0 + r) * n + k0 + c] = buf[c * LDT + r];
    }
    return;
  }
  float* As = buf;
  float* Bs = buf + KT * LDT;
  Quad q;
  float* C = S + int64_t(i0) * n + j0;
  quad_load(q, C, n, bi, bj);
  for (int kc = 0; kc < bk; kc += KT) {
    stage_rows(As, d.Y, n, kc, bk, i0, n);
    stage_rows(Bs, d.Y, n, kc, bk, j0, n);
    __syncthreads();
    quad_mma(q, As, Bs, -1.f);
    __syncthreads();
  }
  quad_store(q, C, n, bi, bj);
}

// inv <- -S with both triangles written (S = inv in place).
__global__ void __launch_bounds__(256) inv_finish_kernel(const InvDesc* __restrict__ desc,
                                                         const int32_t* __restrict__ begin, int count) {
  __shared__ float s[FT][FT + 1];
  const int p = find_problem(begin, count, blockIdx.x);
  const InvDesc& d = desc[p];
  int ti, tj;
  upper_tile(blockIdx.x - begin[p], d.nb64, ti, tj);
  const int64_t n = d.n;
  const int c = threadIdx.x & (FT - 1);
  const int64_t i0 = int64_t(ti) * FT, j0 = int64_t(tj) * FT;
  for (int r = threadIdx.x >> 6; r < FT; r += 4) {
    const int64_t i = i0 + r, j = j0 + c;
    float v = 0.f;
    if (i < n && j < n && i <= j) {
      v = -d.S[i * n + j];
      d.S[i * n + j] = v;
    }
    s[r][c] = v;
  }
  __syncthreads();
  for (int r = threadIdx.x >> 6; r < FT; r += 4) {
    const int64_t j = j0 + r, i = i0 + c;
    if (i < n && j < n && i < j) d.S[j * n + i] = s[c][r];
  }
}

struct InvPlan {
  std::vector<int> order;  // matrices sorted by block count, descending
  std::vector<int32_t> tile_begin, panel_begin, t64_begin;
  std::vector<int32_t> active;  // active[k] = matrices with nb > k
  size_t floats = 0;            // E, Ui, Pn, Y, W for all matrices
  int max_nb = 0;
};

static void plan_inv(int count, const int32_t* n, InvPlan& pl) {
  pl.order.resize(count);
  for (int m = 0; m < count; ++m) pl.order[m] = m;
  std::stable_sort(pl.order.begin(), pl.order.end(), [&](int a, int b) { return n[a] > n[b]; });
  int64_t tiles = 0, panels = 0, t64 = 0;
  pl.tile_begin.resize(count);
  pl.panel_begin.resize(count);
  pl.t64_begin.resize(count);
  for (int q = 0; q < count; ++q) {
    const int nn = n[pl.order[q]];
    const int nb = (nn + TB - 1) / TB, nb64 = (nn + FT - 1) / FT;
    pl.tile_begin[q] = static_cast<int32_t>(tiles);
    pl.panel_begin[q] = static_cast<int32_t>(panels);
    pl.t64_begin[q] = static_cast<int32_t>(t64);
    tiles += int64_t(nb) * (nb + 1) / 2;
    panels += nb - 1;
    t64 += int64_t(nb64) * (nb64 + 1) / 2;
    pl.floats += size_t(3) * TB * TB + size_t(2) * TB * nn;
    if (nb > pl.max_nb) pl.max_nb = nb;
  }
  pl.active.assign(pl.max_nb, 0);
  for (int q = 0; q < count; ++q) {
    const int nb = (n[pl.order[q]] + TB - 1) / TB;
    for (int k = 0; k < nb; ++k) pl.active[k] = q + 1;
  }
}

static size_t inv_ws_bytes(const InvPlan& pl, int count) {
  return align256(sizeof(InvDesc) * count) + 3 * align256(sizeof(int32_t) * count) +
         align256(sizeof(float) * pl.floats);
}

}  // namespace kfac

using namespace kfac;

static kfac_status inv_validate(int32_t count, const int32_t* n) {
  if (count < 0) return fail(KFAC_ERR_INVALID, "count must be >= 0");
  if (count > 0 && !n) return fail(KFAC_ERR_INVALID, "n is NULL");
  for (int m = 0; m < count; ++m)
    if (n[m] < 1 || n[m] > 32768) return fail(KFAC_ERR_INVALID, "n[%d] = %d out of range [1, 32768]", m, n[m]);
  return KFAC_OK;
}

extern "C" kfac_status kfac_invert_workspace(int32_t count, const int32_t* n, size_t* bytes) {
  if (!bytes) return fail(KFAC_ERR_INVALID, "bytes is NULL");
  kfac_status st = inv_validate(count, n);
  if (st) return st;
  if (count == 0) { *bytes = 0; return KFAC_OK; }
  InvPlan pl;
  plan_inv(count, n, pl);
  *bytes = inv_ws_bytes(pl, count);
  return KFAC_OK;
}

extern "C" kfac_status kfac_invert(int32_t count, const int32_t* n, const float* const* mat,
                                   float* const* inv, const float* shift, int32_t* info,
                                   float* const* chol, void* workspace, size_t ws_bytes, void* stream) {
  kfac_status st = inv_validate(count, n);
  if (st) return st;
  if (count == 0) return KFAC_OK;
  if (!mat || !inv || !shift || !info) return fail(KFAC_ERR_INVALID, "NULL pointer argument");
  if (reinterpret_cast<uintptr_t>(info) & 3) return fail(KFAC_ERR_INVALID, "info misaligned");
  for (int m = 0; m < count; ++m) {
    if (!mat[m] || !inv[m]) return fail(KFAC_ERR_INVALID, "matrix %d: NULL pointer", m);
    if ((reinterpret_cast<uintptr_t>(mat[m]) | reinterpret_cast<uintptr_t>(inv[m])) & 3 ||
        (chol && chol[m] && (reinterpret_cast<uintptr_t>(chol[m]) & 3)))
      return fail(KFAC_ERR_INVALID, "matrix %d: misaligned pointer", m);
    if (!(shift[m] == shift[m])) return fail(KFAC_ERR_INVALID, "matrix %d: shift is NaN", m);
  }
  InvPlan pl;
  plan_inv(count, n, pl);
  st = check_device();
  if (st) return st;
  st = check_workspace(workspace, ws_bytes, inv_ws_bytes(pl, count));
  if (st) return st;
  Carver cv(workspace);
  InvDesc* d_desc = cv.take<InvDesc>(count);
  int32_t* d_tile = cv.take<int32_t>(count);
  int32_t* d_panel = cv.take<int32_t>(count);
  int32_t* d_t64 = cv.take<int32_t>(count);
  float* wsf = cv.take<float>(pl.floats);
  std::vector<InvDesc> desc(count);
  size_t off = 0;
  for (int q = 0; q < count; ++q) {
    const int m = pl.order[q];
    InvDesc& d = desc[q];
    d.mat = mat[m];
    d.S = inv[m];
    d.chol = chol ? chol[m] : nullptr;
    d.info = info + m;
    d.n = n[m];
    d.nb = (n[m] + TB - 1) / TB;
    d.nb64 = (n[m] + FT - 1) / FT;
    d.shift = shift[m];
    d.E = wsf + off; off += size_t(TB) * TB;
    d.Ui = wsf + off; off += size_t(TB) * TB;
    d.Pn = wsf + off; off += size_t(TB) * TB;
    d.Y = wsf + off; off += size_t(TB) * n[m];
    d.W = wsf + off; off += size_t(TB) * n[m];
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = upload(d_desc, desc.data(), sizeof(InvDesc) * count, s);
  if (st) return st;
  st = upload(d_tile, pl.tile_begin.data(), sizeof(int32_t) * count, s);
  if (st) return st;
  st = upload(d_panel, pl.panel_begin.data(), sizeof(int32_t) * count, s);
  if (st) return st;
  st = upload(d_t64, pl.t64_begin.data(), sizeof(int32_t) * count, s);
  if (st) return st;
  // grid sizes for the active prefix [0, a): begin[a] or the grand total
  auto grid_of = [&](const std::vector<int32_t>& begin, int a, auto per) -> unsigned {
    if (a < count) return static_cast<unsigned>(begin[a]);
    return static_cast<unsigned>(begin[count - 1] + per(pl.order[count - 1]));
  };
  auto tiles_of = [&](int m) { int nb = (n[m] + TB - 1) / TB; return nb * (nb + 1) / 2; };
  auto panels_of = [&](int m) { return (n[m] + TB - 1) / TB - 1; };
  auto t64_of = [&](int m) { int nb = (n[m] + FT - 1) / FT; return nb * (nb + 1) / 2; };

  KFAC_LAUNCH(K_INV_PREP, inv_prep_kernel, dim3(grid_of(pl.t64_begin, count, t64_of)), dim3(256), 0, s,
              d_desc, d_t64, count);
  KFAC_CHECK_LAUNCH("inv_prep_kernel");
  for (int k = 0; k < pl.max_nb; ++k) {
    const int a = pl.active[k];
    KFAC_LAUNCH(K_INV_PIVOT, inv_pivot_kernel, dim3(a), dim3(1024), 0, s, d_desc, k);
    KFAC_CHECK_LAUNCH("inv_pivot_kernel");
    const unsigned panels = grid_of(pl.panel_begin, a, panels_of);
    if (panels) {
      KFAC_LAUNCH(K_INV_PANEL, inv_panel_kernel, dim3(panels), dim3(256), 0, s, d_desc, d_panel, a, k);
      KFAC_CHECK_LAUNCH("inv_panel_kernel");
    }
    KFAC_LAUNCH(K_INV_UPDATE, inv_update_kernel, dim3(grid_of(pl.tile_begin, a, tiles_of)), dim3(256), 0, s,
                d_desc, d_tile, a, k);
    KFAC_CHECK_LAUNCH("inv_update_kernel");
  }
  KFAC_LAUNCH(K_INV_FINISH, inv_finish_kernel, dim3(grid_of(pl.t64_begin, count, t64_of)), dim3(256), 0, s,
              d_desc, d_t64, count);
  KFAC_CHECK_LAUNCH("inv_finish_kernel");
  return KFAC_OK;
}
