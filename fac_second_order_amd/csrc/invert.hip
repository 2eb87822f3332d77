// Batched damped inverses (F + s I)^-1 of symmetric positive definite factors.
// Osawa et al. (CVPR 2019), Section 3.2, eq. (6): the inverse of the Kronecker
// product is the Kronecker product of the factors' inverses, so each factor is
// inverted on its own; damping adds s to the diagonal of each factor.
//
// Method: a blocked right-looking Cholesky factorisation M = U^T U (block 128, no
// pivoting) in which every block step is also applied to the rows and columns
// that were already eliminated, so the inverse is assembled in the same sweep
// (the symmetric Gauss-Jordan form of the Cholesky inverse). With S the working
// matrix (upper triangle in 128-blocks) and k the pivot block, one step is
//   pivot:  U_kk = chol(S_kk) and E = U_kk^-T, by one workgroup with the block in
//           registers: per column, one LDS broadcast of the scaled pivot row and one
//           barrier; rows above the pivot are finished and skipped;
//   panel:  for every column block j != k: V_j = S_kj, Y_j = E V_j (the Cholesky
//           row panel U_kj when j > k) and W_j = E^T Y_j = P^-1 V_j, on MFMA, with
//           S_kj = W_j (S_jk = W_j^T for j < k) written in place and Y_j kept in a
//           row-major panel buffer; the block j = k writes S_kk = -E^T E = -P^-1;
//   update: S_ij -= Y_i^T Y_j for all upper tiles i, j != k (fp32 MFMA).
// The update works on the square root Y of V^T P^-1 V, so its rounding errors scale
// with |Y|^2 rather than with |V| |P^-1 V| (which an explicit P^-1 would give).
// Steps are taken in pairs (k, k+1): after panel k only the tiles of block row
// k+1 take step k's update (row update), then pivot and panel k+1 run, and one
// update applies both steps, S_ij -= [Y_i; Y'_i]^T [Y_j; Y'_j], a rank-256 product
// that reads and writes each tile once for two steps (tiles in block row k take
// only step k+1's half). After the last step S = -M^-1; the finish kernel negates
// it and writes both triangles. All matrices of a call step together: they are
// ordered by block count, so the ones still active at step k are a prefix.
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
  float* Y;        // [2*TB][ldy] Y panels of steps k (rows 0..) and k+1 (rows TB..)
  int32_t n, nb;
  float shift;
  int32_t nb64;    // 64-wide blocks (prep/finish tiles)
  int32_t ldy;     // n rounded up to a multiple of 4 (16-byte rows)
  int32_t pad_;
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
  if (ti == 0 && tj == 0 && threadIdx.x == 0) *gp(d.info) = 0;
  if (d.mat == d.S) {  // in place: only the diagonal changes
    if (ti == tj && threadIdx.x < FT) {
      const int64_t i = int64_t(ti) * FT + threadIdx.x;
      if (i < n) gp(d.S)[i * n + i] += d.shift;
    }
    return;
  }
  const int c = threadIdx.x & (FT - 1);
  const int64_t j = int64_t(tj) * FT + c;
  for (int r = threadIdx.x >> 6; r < FT; r += 4) {
    const int64_t i = int64_t(ti) * FT + r;
    if (i < n && j < n && i <= j) {
      float v = gp(d.mat)[i * n + j];
      if (i == j) v += d.shift;
      gp(d.S)[i * n + j] = v;
    }
  }
}

// Cholesky of the pivot block P (bk x bk, upper triangle in S) and E = U^-T, by the
// PT threads of one block. Wave w holds rows RPW*w .. RPW*w+RPW-1 and lane l
// columns 2l, 2l+1 of a combined matrix whose strict upper triangle becomes U,
// strict lower triangle E and diagonal 1/U_ii. Scalar step kk: the pivot row is
// scaled, r = M_kk^-1/2 * M_k. with r_kk = M_kk^-1/2; every row i > kk clears its
// entry in column kk and loses u_i * r with u_i = r_i; rows <= kk are final.
// Columns are taken GP at a time: the wave that owns rows c0..c0+GP-1 runs the GP
// steps on them in registers (broadcasts by readlane, no barrier), publishes the GP
// scaled rows through LDS, and after one barrier every later row applies the GP
// updates. Waves whose rows are all final skip the update. Padding rows/columns
// (>= bk) hold the identity and stay unchanged. Writes E and U^-1 = E^T
// (row-major, TB x TB) to the workspace, U into chol when asked, and the 1-based
// failing column into info.
constexpr int PT = 512;           // threads of the pivot kernel
constexpr int NW = PT / 64;       // waves
constexpr int RPW = TB / NW;      // rows per wave (contiguous)
constexpr int GP = 4;             // pivot columns per barrier

__device__ __forceinline__ float lane_bcast(float v, int src_lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src_lane));
}

// The owner wave's GP steps on its rows QQ*GP .. QQ*GP+GP-1 (columns c0 ..).
template <int QQ>
__device__ __forceinline__ void pivot_group(float2 (&M)[RPW], int c0, int gcnt, int lane,
                                            float (*prow)[TB], float* dval, float* diagU) {
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    if (g < gcnt) {
      const int a = c0 + g, al = a >> 1;
      const bool aodd = a & 1;
      const float2 m = M[QQ * GP + g];
      const float piv = lane_bcast(aodd ? m.y : m.x, al);
      const float rs = rsqrtf(piv);
      float2 sc = make_float2(m.x * rs, m.y * rs);
      if (lane == al) {
        if (aodd) sc.y = rs; else sc.x = rs;
      }
      M[QQ * GP + g] = sc;
      reinterpret_cast<float2*>(prow[g])[lane] = sc;
      if (lane == 0) {
        dval[g] = piv;
        diagU[a] = piv * rs;
      }
#pragma unroll
      for (int g2 = g + 1; g2 < GP; ++g2) {
        if (g2 < gcnt) {
          const int b = c0 + g2;
          const float u = lane_bcast((b & 1) ? sc.y : sc.x, b >> 1);
          float2 mb = M[QQ * GP + g2];
          if (lane == al) {
            if (aodd) mb.y = 0.f; else mb.x = 0.f;
          }
          mb.x = fmaf(-u, sc.x, mb.x);
          mb.y = fmaf(-u, sc.y, mb.y);
          M[QQ * GP + g2] = mb;
        }
      }
    }
  }
}

__global__ void __launch_bounds__(PT) inv_pivot_kernel(const InvDesc* __restrict__ desc, int k) {
  const InvDesc& d = desc[blockIdx.x];
  const int n = d.n, k0 = k * TB, bk = min(TB, n - k0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, scalar
  __shared__ __attribute__((aligned(16))) float prow[2][GP][TB];  // scaled pivot rows
  __shared__ __attribute__((aligned(16))) float dval[2][GP];
  __shared__ float diagU[TB];
  __shared__ float L[TB * LDT];

  float2 M[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int i = RPW * w + r;
    const int j0 = 2 * lane, j1 = 2 * lane + 1;
    float a = (i == j0) ? 1.f : 0.f, b = (i == j1) ? 1.f : 0.f;
    if (i < bk && j0 < bk) a = gp(d.S)[int64_t(k0 + min(i, j0)) * n + k0 + max(i, j0)];
    if (i < bk && j1 < bk) b = gp(d.S)[int64_t(k0 + min(i, j1)) * n + k0 + max(i, j1)];
    M[r] = make_float2(a, b);
  }
  int failed = 0;
  for (int c0 = 0; c0 < bk; c0 += GP) {
    const int buf = (c0 / GP) & 1;
    const int gcnt = min(GP, bk - c0);
    if (w == c0 / RPW) {
      const int q = (c0 % RPW) / GP;
      if (q == 0) pivot_group<0>(M, c0, gcnt, lane, prow[buf], dval[buf], diagU);
      else if (q == 1) pivot_group<1>(M, c0, gcnt, lane, prow[buf], dval[buf], diagU);
      else if (q == 2) pivot_group<2>(M, c0, gcnt, lane, prow[buf], dval[buf], diagU);
      else pivot_group<3>(M, c0, gcnt, lane, prow[buf], dval[buf], diagU);
    }
    __syncthreads();
    {
      const float4 pv = *reinterpret_cast<const float4*>(dval[buf]);
      const float pp[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
      for (int g = GP - 1; g >= 0; --g)  // keep the first bad column
        if (g < gcnt && (!(pp[g] > 0.f) || !isfinite(pp[g]))) failed = c0 + g + 1;
    }
    if (failed) break;  // same decision in every thread
    const int last = c0 + gcnt - 1;  // rows > last take the GP updates
    if (RPW * w + RPW - 1 > last) {
      float2 rjs[GP];
      float us[GP][RPW];  // all multipliers first: one LDS round trip
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        rjs[g] = reinterpret_cast<const float2*>(prow[buf][g])[lane];
#pragma unroll
        for (int q = 0; q < RPW / 4; ++q) {
          const float4 x = reinterpret_cast<const float4*>(prow[buf][g] + RPW * w)[q];
          us[g][4 * q] = x.x; us[g][4 * q + 1] = x.y; us[g][4 * q + 2] = x.z; us[g][4 * q + 3] = x.w;
        }
      }
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        if (g < gcnt) {
          const int a = c0 + g, al = a >> 1;
          const bool aodd = a & 1;
          const float2 rj = rjs[g];
          const float* u = us[g];
          const bool mycol = lane == al;
#pragma unroll
          for (int r = 0; r < RPW; ++r) {
            if (RPW * w + r > last) {
              float2 m = M[r];
              if (mycol) {
                if (aodd) m.y = 0.f; else m.x = 0.f;
              }
              m.x = fmaf(-u[r], rj.x, m.x);
              m.y = fmaf(-u[r], rj.y, m.y);
              M[r] = m;
            }
          }
        }
      }
    }
  }
  // E (strict lower + diagonal) into L, then coalesced writes of E and E^T
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int i = RPW * w + r;
    const float2 m = M[r];
    L[i * LDT + 2 * lane] = (2 * lane <= i) ? m.x : 0.f;
    L[i * LDT + 2 * lane + 1] = (2 * lane + 1 <= i) ? m.y : 0.f;
    if (d.chol) {
      if (i < 2 * lane && 2 * lane < bk) gp(d.chol)[int64_t(k0 + i) * n + k0 + 2 * lane] = m.x;
      if (i < 2 * lane + 1 && 2 * lane + 1 < bk) gp(d.chol)[int64_t(k0 + i) * n + k0 + 2 * lane + 1] = m.y;
    }
  }
  __syncthreads();
  for (int e = tid; e < TB * TB; e += PT) {
    const int i = e / TB, j = e % TB;
    gp(d.E)[e] = L[i * LDT + j];
    gp(d.Ui)[e] = L[j * LDT + i];
  }
  if (d.chol)
    for (int i = tid; i < bk; i += PT) gp(d.chol)[int64_t(k0 + i) * n + k0 + i] = diagU[i];
  if (failed && tid == 0 && *gp(d.info) == 0) *gp(d.info) = k0 + failed;
}

// Panel of step k into buffer slot `slot` (Y rows slot*TB ..): for column block
// j != k, Y_j = E V_j and W_j = E^T Y_j, with W_j written into S in place; column
// block j = k writes S_kk = -E^T E.
__global__ void __launch_bounds__(256) inv_panel_kernel(const InvDesc* __restrict__ desc,
                                                        const int32_t* __restrict__ begin,
                                                        int count, int k, int slot) {
  const int p = find_problem(begin, count, blockIdx.x);
  const InvDesc& d = desc[p];
  const int j = blockIdx.x - begin[p];
  const int n = d.n, k0 = k * TB, bk = min(TB, n - k0);
  const int j0 = j * TB, bj = min(TB, n - j0);
  __shared__ __attribute__((aligned(16))) float lds[4 * CHUNK];
  __shared__ __attribute__((aligned(16))) float Ys[TB * LDP];

  Quad q;
  quad_zero(q);
  const Operand Eop = op_rows(d.E, TB, bk, 0, bk);   // A[p][m] = E[p][m] = Ui[m][p]
  if (j == k) {  // S_kk = -E^T E (upper triangle)
    quad_gemm(q, Eop, Eop, bk, -1.f, lds);
    quad_store_upper(q, d.S + int64_t(k0) * n + k0, n, bk);
    return;
  }
  const Operand Uop = op_rows(d.Ui, TB, bk, 0, bk);  // A[p][m] = Ui[p][m] = E[m][p]
  const Operand V = j > k ? op_rows(d.S + int64_t(k0) * n + j0, n, bk, 0, bj)    // V = S_kj
                          : op_cols(d.S + int64_t(j0) * n + k0, n, bk, 0, bj);   // V = S_jk^T
  quad_gemm(q, Uop, V, bk, 1.f, lds);
  quad_store(q, d.Y + int64_t(slot) * TB * d.ldy + j0, d.ldy, bk, bj);
  if (d.chol && j > k) quad_store(q, d.chol + int64_t(k0) * n + j0, n, bk, bj);
  quad_to_lds(q, Ys, LDP);  // rows >= bk are zero (their A columns were zero)
  quad_zero(q);
  __syncthreads();
  quad_gemm_lds_b(q, Eop, Ys, LDP, bk, 1.f, lds);
  if (j > k) quad_store(q, d.S + int64_t(k0) * n + j0, n, bk, bj);        // S_kj = W_j
  else quad_store_t(q, d.S + int64_t(j0) * n + k0, n, bk, bj, lds);       // S_jk = W_j^T
}

// Update of step k: S_ij -= Y_i^T Y_j over the upper 128-tile of row blocks i, j,
// with rows [kb, ke) of the stacked panel buffer.
__device__ __forceinline__ void update_tile(const InvDesc& d, int ti, int tj, int kb, int ke, float* lds) {
  const int n = d.n, i0 = ti * TB, j0 = tj * TB;
  const int bi = min(TB, n - i0), bj = min(TB, n - j0);
  Quad q;
  float* C = d.S + int64_t(i0) * n + j0;
  quad_load(q, C, n, bi, bj);
  // panel rows are 16-byte aligned with pitch ldy = n rounded up to 4 (workspace carve-out)
  const float* Y = d.Y + int64_t(kb) * d.ldy;
  quad_gemm<true>(q, op_rows(Y, d.ldy, ke - kb, i0, n), op_rows(Y, d.ldy, ke - kb, j0, n), ke - kb, -1.f, lds);
  quad_store(q, C, n, bi, bj);
}

// Update after step k, or after steps k and k+1 when `pair` is set and the matrix
// has block k+1: every upper tile outside block row k+1 (k when unpaired) takes the
// rank-(bk + bk1) product of both steps, tiles in block row k only step k+1's half.
__global__ void __launch_bounds__(256) inv_update_kernel(const InvDesc* __restrict__ desc,
                                                         const int32_t* __restrict__ begin,
                                                         int count, int k, int total, int pair) {
  const int v = xcd_virtual(blockIdx.x, gridDim.x, total);
  if (v < 0) return;
  const int p = find_problem(begin, count, v);
  const InvDesc& d = desc[p];
  int ti, tj;
  upper_tile(v - begin[p], d.nb, ti, tj);
  const bool paired = pair && k + 1 < d.nb;
  const int kx = paired ? k + 1 : k;  // written by its panel kernel
  if (ti == kx || tj == kx) return;
  const int bk = min(TB, d.n - k * TB);
  int kb = 0, ke = bk;
  if (paired) {
    kb = (ti == k || tj == k) ? TB : 0;
    ke = TB + min(TB, d.n - (k + 1) * TB);
  }
  __shared__ __attribute__((aligned(16))) float lds[4 * CHUNK];
  update_tile(d, ti, tj, kb, ke, lds);
}

// Step k's update of block row k+1 before its pivot (paired steps): the tiles
// (k+1, j) for j != k, stored as upper tiles (min, max).
__global__ void __launch_bounds__(256) inv_rowupd_kernel(const InvDesc* __restrict__ desc,
                                                         const int32_t* __restrict__ begin,
                                                         int count, int k) {
  const int p = find_problem(begin, count, blockIdx.x);
  const InvDesc& d = desc[p];
  const int j = blockIdx.x - begin[p];
  if (j == k) return;
  __shared__ __attribute__((aligned(16))) float lds[4 * CHUNK];
  update_tile(d, min(j, k + 1), max(j, k + 1), 0, TB, lds);
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
      v = -gp(d.S)[i * n + j];
      gp(d.S)[i * n + j] = v;
    }
    s[r][c] = v;
  }
  __syncthreads();
  for (int r = threadIdx.x >> 6; r < FT; r += 4) {
    const int64_t j = j0 + r, i = i0 + c;
    if (i < n && j < n && i < j) gp(d.S)[j * n + i] = s[c][r];
  }
}

struct InvPlan {
  std::vector<int> order;  // matrices sorted by block count, descending
  std::vector<int32_t> tile_begin, panel_begin, t64_begin;
  std::vector<int32_t> active;  // active[k] = matrices with nb > k
  size_t floats = 0;            // E, Ui, Y for all matrices
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
    panels += nb;
    t64 += int64_t(nb64) * (nb64 + 1) / 2;
    pl.floats += size_t(2) * TB * TB + size_t(2) * TB * ((nn + 3) / 4 * 4);
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
    d.ldy = (n[m] + 3) / 4 * 4;
    d.Y = wsf + off; off += size_t(2) * TB * d.ldy;
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
  auto panels_of = [&](int m) { return (n[m] + TB - 1) / TB; };
  auto t64_of = [&](int m) { int nb = (n[m] + FT - 1) / FT; return nb * (nb + 1) / 2; };

  KFAC_LAUNCH(K_INV_PREP, inv_prep_kernel, dim3(grid_of(pl.t64_begin, count, t64_of)), dim3(256), 0, s,
              d_desc, d_t64, count);
  KFAC_CHECK_LAUNCH("inv_prep_kernel");
  auto update = [&](int a, int k, int pair) -> kfac_status {
    const unsigned ut = grid_of(pl.tile_begin, a, tiles_of);
    KFAC_LAUNCH(K_INV_UPDATE, inv_update_kernel, dim3(xcd_grid(ut)), dim3(256), 0, s, d_desc, d_tile, a, k,
                static_cast<int>(ut), pair);
    KFAC_CHECK_LAUNCH("inv_update_kernel");
    return KFAC_OK;
  };
  for (int k = 0; k < pl.max_nb; k += 2) {  // steps in pairs
    const int a0 = pl.active[k];
    const int a1 = k + 1 < pl.max_nb ? pl.active[k + 1] : 0;
    KFAC_LAUNCH(K_INV_PIVOT, inv_pivot_kernel, dim3(a0), dim3(PT), 0, s, d_desc, k);
    KFAC_CHECK_LAUNCH("inv_pivot_kernel");
    KFAC_LAUNCH(K_INV_PANEL, inv_panel_kernel, dim3(grid_of(pl.panel_begin, a0, panels_of)), dim3(256), 0, s,
                d_desc, d_panel, a0, k, 0);
    KFAC_CHECK_LAUNCH("inv_panel_kernel");
    if (a1 > 0) {
      const unsigned pg = grid_of(pl.panel_begin, a1, panels_of);
      KFAC_LAUNCH(K_INV_ROWUPD, inv_rowupd_kernel, dim3(pg), dim3(256), 0, s, d_desc, d_panel, a1, k);
      KFAC_CHECK_LAUNCH("inv_rowupd_kernel");
      KFAC_LAUNCH(K_INV_PIVOT, inv_pivot_kernel, dim3(a1), dim3(PT), 0, s, d_desc, k + 1);
      KFAC_CHECK_LAUNCH("inv_pivot_kernel");
      KFAC_LAUNCH(K_INV_PANEL, inv_panel_kernel, dim3(pg), dim3(256), 0, s, d_desc, d_panel, a1, k + 1, 1);
      KFAC_CHECK_LAUNCH("inv_panel_kernel");
    }
    if ((st = update(a0, k, 1))) return st;
  }
  KFAC_LAUNCH(K_INV_FINISH, inv_finish_kernel, dim3(grid_of(pl.t64_begin, count, t64_of)), dim3(256), 0, s,
              d_desc, d_t64, count);
  KFAC_CHECK_LAUNCH("inv_finish_kernel");
  return KFAC_OK;
}
