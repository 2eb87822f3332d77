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
// Steps are taken in groups of GS (kg .. kg+GS-1) with one update per group: before
// pivot k of a group, block row k takes the group's earlier steps (row update; the
// other tiles of the row are extra blocks of that pivot's launch; of the diagonal
// block, which the pivot needs first, the pivot applies only step k-1: each earlier
// step kg+t-1 reached it as an extra block of panel launch kg+t), then panel k writes
// its Y into slot k - kg of the panel buffer; after the last step one update applies
// the whole group, S_ij -= [Y_i; Y'_i; ..]^T [Y_j; Y'_j; ..], a rank-(GS*TB) product that reads and
// writes each tile once per group (tiles in a row of the group take only the steps
// after that row's own). After the last step S = -M^-1; the finish kernel negates
// it and writes both triangles. All matrices of a call step together: they are
// ordered by order n, so the ones still active at step k are a prefix.
// An order n = 128m + 1 (a factor with its bias column) would end with a 1-wide block:
// a whole pivot, panel and rank-1 pass over the matrix for one column. Its last
// column is instead taken as a bordered step: the sweep runs m block steps (which
// still update the last column, in the group updates as a matrix-vector product
// rather than as 1-wide tiles), inv_border_kernel saves the last column v and
// pivot p, and the finish applies the step as it writes the inverse (with
// y = p^-1/2 v: S_ij - y_i y_j inside, p^-1 v on the border, -p^-1 at the corner).
#include <algorithm>

#include "tile_f32.hpp"

namespace kfac {

struct InvDesc {
  const float* mat;
  float* S;        // working matrix = the output buffer
  float* chol;     // optional U output (nullptr)
  int32_t* info;   // this matrix's info entry
  float* E;        // [TB][TB]  E = U_kk^-T, row-major (lower triangular; U_kk^-1 = E^T)
  float* P;        // [TB][TB]  P^-1 = E^T E (full)
  float* Y;        // [GS*TB][ldy] Y panels of the steps of a group (step kg+s in rows s*TB..)
  int32_t n, nb;
  int32_t ns;      // block steps of the sweep: nb, or nb - 1 with a bordered last column
  float shift;
  int32_t nb64;    // 64-wide blocks (prep/finish tiles)
  int32_t ldy;     // n rounded up to a multiple of 4 (16-byte rows)
  int32_t pad_;
};

constexpr int FT = 64;  // prep/finish tile edge

// Block steps of the sweep for order n: the last column of an order 128m + 1 (m >= 1)
// is a bordered step of the finish instead of a 1-wide block step.
__host__ __device__ inline int block_steps(int n) {
  return (n > TB && n % TB == 1) ? n / TB : (n + TB - 1) / TB;
}
// Block steps per update launch (a group): the update of a group applies all its
// steps at once as one rank-(G*TB) product.
#ifndef KFAC_INV_GROUP
#define KFAC_INV_GROUP 6
#endif
constexpr int GS = KFAC_INV_GROUP;
static_assert(GS >= 1 && GS <= 8, "group size");

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

// In-place damping when every matrix is inverted in place: one block per 128 rows
// adds the shift to the diagonal (and block 0 of a matrix zeroes its info), instead of
// a grid over all prep tiles in which only the diagonal ones have work.
__global__ void __launch_bounds__(TB) inv_damp_kernel(const InvDesc* __restrict__ desc,
                                                      const int32_t* __restrict__ begin, int count) {
  const int p = find_problem(begin, count, blockIdx.x);
  const InvDesc& d = desc[p];
  const int kb = blockIdx.x - begin[p];
  if (kb == 0 && threadIdx.x == 0) *gp(d.info) = 0;
  const int64_t i = int64_t(kb) * TB + threadIdx.x;
  if (i < d.n) gp(d.S)[i * d.n + i] += d.shift;
}

// Pivot of step k: U = chol(P) and E = U^-T of the pivot block P (bk x bk, upper
// triangle in S; padding rows and columns hold the identity), then P^-1 = E^T E.
// One 512-thread block keeps the combined matrix M in LDS: its upper triangle
// becomes U, its lower triangle (with the diagonal) E. In scalar form, step c
// scales row c by p^-1/2 (p = M_cc) and gives its diagonal the value p^-1/2
// (= E_cc), so row c becomes r; every later row i > c replaces its column-c entry
// by 0 and then subtracts u_i r with u_i = r_i. The columns are taken in four
// sub-steps J of 32 (block indices I, K in 0..3):
//   a: wave 0 runs the 32 scalar steps on the diagonal block M_JJ in registers
//      (pivot rows broadcast through LDS), giving U_JJ and E_JJ;
//   b: the rest of block row J is multiplied by E_JJ (MFMA): M_JK <- E_JJ M_JK,
//      which makes U_JK (K > J) and E_JK (K < J);
//   c: every later block row I > J subtracts M_JI^T times block row J, on the
//      blocks it still needs: K > J with I <= K (the trailing upper triangle),
//      K < J (the E part) and K = J, which becomes -M_JI^T E_JJ.
// The lower blocks right of the current sub-step are never read before their own
// sub-step overwrites them, so they start as zero. Writes E (row-major, TB x TB; its
// transpose is U^-1) and P^-1 to the workspace (the operands of the panel), S_kk = -P^-1, U into
// chol when asked, and the 1-based failing column into info.
// 16 bytes at a 4-byte aligned address (rows of an odd order start anywhere)
typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));
constexpr int PT = 512;           // threads of the pivot kernel
constexpr int SB = 32;            // sub-step width
constexpr int MLD = TB + 4;       // LDS pitch of M
constexpr int ELD = SB + 1;       // LDS pitch of the 32x32 E_JJ copies (odd: read along rows and columns)

// acc[m][n] += sign * sum_p a[p*lda + m] * b[p*ldb + n] for p < 32 (one wave, LDS).
// Accumulator register e of lane l holds element (8*(e/4) + 4*(l/32) + e%4, l%32).
__device__ __forceinline__ void mma32(v16f& acc, const float* a, int lda, const float* b, int ldb,
                                      float sign, int lane) {
  const int ml = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int k = 0; k < SB; k += 2) {
    const float av = a[(k + kh) * lda + ml] * sign;
    const float bv = b[(k + kh) * ldb + ml];
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
  }
}
// The same with the A operand read transposed: element (m, p) = a[m*lda + p].
__device__ __forceinline__ void mma32_at(v16f& acc, const float* a, int lda, const float* b, int ldb, int lane) {
  const int ml = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int k = 0; k < SB; k += 2) {
    const float av = a[ml * lda + k + kh];
    const float bv = b[(k + kh) * ldb + ml];
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
  }
}
__device__ __forceinline__ int acc_row(int e, int lane) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

__device__ __forceinline__ float lane_bcast(float v, int src_lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src_lane));
}

// Scalar steps on the 32x32 diagonal block at blk (pitch MLD) by one wave: lane
// j + 32h holds rows t = 2q + h (q = 0..15) of column j, so both halves of the
// wave share every step's work. Publishing row c: the lanes holding it scale it
// into the pivot row r (diagonal entry p^-1/2 = E_cc) and write it to LDS split by
// row parity (urow[t & 1][t >> 1] = r_t). Step c: with its column's r_j and the
// r_t of its rows, a lane updates the rows t > c (column c cleared, then
// M_tj -= r_t r_j). Row c+1 is updated and published first, and the broadcast of
// step c+1 is read before the remaining rows of step c are updated, so LDS latency
// overlaps arithmetic (LDS operations of one wave complete in order). Writes the
// block back, E_JJ to ej (rows, lower with diagonal) and its transpose to uil
// (global, row-major, pitch TB), U_cc to diagU; returns the first 1-based failing step or 0.
__device__ __forceinline__ int chol32(float* blk, float* ej, KG float* eg, float* diagU,
                                      float (*urow)[SB / 2], int lane) {
  const int j = lane & 31, h = lane >> 5;
  float d[SB / 2];
#pragma unroll
  for (int q = 0; q < SB / 2; ++q) d[q] = blk[(2 * q + h) * MLD + j];
  int failed = 0;
  float ujj = 0.f;
  auto publish = [&](int c) {  // row c is final: scale it into the pivot row
    const int hc = c & 1, qc = c >> 1;
    const float p = lane_bcast(d[qc], c + 32 * hc);
    if (failed == 0 && !(p > 0.f && isfinite(p))) failed = c + 1;
    const float rs = rsqrtf(p);
    if (h == hc) {
      const bool jc = j == c;
      const float r = jc ? rs : d[qc] * rs;
      if (jc) ujj = p * rs;
      d[qc] = r;
      urow[j & 1][j >> 1] = r;
    }
  };
  auto fetch = [&](float& rj, float (&u)[SB / 2]) {
    rj = urow[j & 1][j >> 1];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 x = reinterpret_cast<const float4*>(urow[h])[v];
      u[4 * v] = x.x; u[4 * v + 1] = x.y; u[4 * v + 2] = x.z; u[4 * v + 3] = x.w;
    }
  };
  float rj, u[SB / 2];
  publish(0);
  __builtin_amdgcn_wave_barrier();
  fetch(rj, u);
#pragma unroll
  for (int c = 0; c < SB; ++c) {
    if (c + 1 < SB) {
      const bool jc = j == c;
      const int q1 = (c + 1) >> 1, h1 = (c + 1) & 1;
      if (h == h1) d[q1] = fmaf(-u[q1], rj, jc ? 0.f : d[q1]);  // row c+1
      __builtin_amdgcn_wave_barrier();
      publish(c + 1);
      __builtin_amdgcn_wave_barrier();
      float rj2, u2[SB / 2];
      fetch(rj2, u2);  // step c+1's broadcast, in flight during the rest of step c
      __builtin_amdgcn_wave_barrier();
      if (c & 1) {  // slot q1 of the other half holds row c+2
        if (h == 1) d[q1] = fmaf(-u[q1], rj, jc ? 0.f : d[q1]);
      }
#pragma unroll
      for (int q = q1 + 1; q < SB / 2; ++q) d[q] = fmaf(-u[q], rj, jc ? 0.f : d[q]);
      rj = rj2;
#pragma unroll
      for (int q = 0; q < SB / 2; ++q) u[q] = u2[q];
    }
  }
  if (h == (j & 1)) diagU[j] = ujj;
#pragma unroll
  for (int q = 0; q < SB / 2; ++q) {
    const int t = 2 * q + h;
    blk[t * MLD + j] = d[q];
    const float e = j <= t ? d[q] : 0.f;  // E_JJ[t][j]
    ej[t * ELD + j] = e;
    eg[t * TB + j] = e;
  }
  return failed;
}

// Update of step k: S_ij -= Y_i^T Y_j over the upper 128-tile of row blocks i, j,
// with rows [kb, ke) of the stacked panel buffer.
// 512-thread blocks (the oct engine).
__device__ __forceinline__ void update_tile(const InvDesc& d, int ti, int tj, int kb, int ke, float* lds) {
  const int n = d.n, i0 = ti * TB, j0 = tj * TB;
  const int bi = min(TB, n - i0), bj = min(TB, n - j0);
  Oct o;
  float* C = d.S + int64_t(i0) * n + j0;
  oct_load(o, C, n, bi, bj);
  // panel rows are 16-byte aligned with pitch ldy = n rounded up to 4 (workspace carve-out)
  const float* Y = d.Y + int64_t(kb) * d.ldy;
  oct_gemm(o, op_rows(Y, d.ldy, ke - kb, i0, n), op_rows(Y, d.ldy, ke - kb, j0, n), ke - kb, -1.f, lds);
  oct_store(o, C, n, bi, bj);
}

// Pivot of step k. Sub-step J runs, after barriers: A (wave 0 factors the diagonal
// block while waves 1..7 finish sub-step J-1's updates outside block row J),
// B (block row J times E_JJ), C (sub-step J's update of the next diagonal block
// only, which A of J+1 needs first).
// Blocks [0, a) are the pivots of matrices 0..a-1. For step k = kg + pre of a group
// starting at kg, the updates of the group's earlier steps kg..k-1 have not reached
// block row k yet, except that the panel launches applied steps kg..k-2 to the
// diagonal block: each pivot first applies step k-1 to its own diagonal block (S_kk -=
// Y^T Y over panel rows [(pre-1)*TB, pre*TB)), and blocks [a, a + rows) apply them all to the other
// tiles (k, j) of the row, which nothing else in the launch reads or writes; they find
// their tile through the panel offsets `begin`. A tile (k, j) with j = kg + s', s' <
// pre, was rewritten by the panel of step j and takes only the steps after it.
__global__ void __launch_bounds__(PT) inv_pivot_kernel(const InvDesc* __restrict__ desc,
                                                       const int32_t* __restrict__ begin, int a, int k,
                                                       int pre, int rows) {
  // 80.5 KB in all, at most half the LDS of a compute unit, so that a pivot block fits
  // next to one block of the other matrix kernels (67.6 KB at most): E and P^-1 go
  // straight to global memory, and the staging planes of the diagonal pre-update share
  // their space with the two E_JJ buffers.
  __shared__ __attribute__((aligned(16))) float M[TB * MLD];
  __shared__ __attribute__((aligned(16))) float XU[X3_GRAM_LDS_BYTES / 4];
  static_assert(X3_GRAM_LDS_BYTES >= 2 * SB * ELD * 4, "E_JJ copies do not fit the shared space");
  float (*EJ)[SB * ELD] = reinterpret_cast<float (*)[SB * ELD]>(XU);
  __shared__ __attribute__((aligned(16))) float urow[2][SB / 2];
  __shared__ float diagU[TB];
  if (static_cast<int>(blockIdx.x) >= a) {  // a tile of block row k (M is the staging LDS)
    const int t = blockIdx.x - a;
    if (t >= rows) return;
    const int p = find_problem(begin, a, t);
    const int j = t - begin[p];
    const int kg = k - pre;
    const int kb = (j >= kg && j < k) ? (j - kg + 1) * TB : 0, ke = pre * TB;
    if (j == k || kb >= ke) return;
    update_tile(desc[p], min(j, k), max(j, k), kb, ke, M);
    return;
  }
  const InvDesc& d = desc[blockIdx.x];
  const int n = d.n, k0 = k * TB, bk = min(TB, n - k0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, scalar

  {  // thread: column tid % 128, rows tid / 128 + 4q; all 32 loads in flight first
    const int j = tid & (TB - 1), r0 = tid >> 7;
    const KG float* src = gp(d.S) + int64_t(k0) * n + k0 + j;
    float v[TB / 4];
#pragma unroll
    for (int q = 0; q < TB / 4; ++q) {
      const int i = r0 + 4 * q;
      v[q] = (i <= j && j < bk) ? src[int64_t(i) * n] : (i == j ? 1.f : 0.f);
    }
#pragma unroll
    for (int q = 0; q < TB / 4; ++q) M[(r0 + 4 * q) * MLD + j] = v[q];
  }
  if (pre) {  // S_kk -= Y_k^T Y_k on the upper triangle, XU as the staging planes
    __syncthreads();
    Oct o;  // -S_kk + Y^T Y, the exact negation of S_kk - Y^T Y summed the same way
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) o.c[b][e] = -M[oct_row(lane, e) * MLD + oct_col(lane, b)];
    // panel rows [(pre-1)*TB, pre*TB): step k-1 (a full block: a matrix's narrow
    // last step is never followed by a pivot)
    const float* Y = d.Y + int64_t(pre - 1) * TB * d.ldy;
    oct_gram(o, op_rows(Y, d.ldy, TB, k0, n), reinterpret_cast<__bf16*>(XU));  // ends with a barrier
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = oct_row(lane, e), c = oct_col(lane, b);
        if (r <= c && c < bk) M[r * MLD + c] = -o.c[b][e];
      }
  }
  __syncthreads();

  // one 32x32 block of sub-step J's trailing update: (I, K) -= M_JI^T B_K, with
  // B_K = M_JK, or E_JJ for K = J (the block starting from zero)
  auto update_block = [&](int J, int I, int K) {
    const float* rowJ = M + J * SB * MLD;
    float* C = M + I * SB * MLD + K * SB;
    v16f acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = K == J ? 0.f : C[acc_row(e, lane) * MLD + (lane & 31)];
    const float* B = K == J ? EJ[J & 1] : rowJ + K * SB;
    mma32(acc, rowJ + I * SB, MLD, B, K == J ? ELD : MLD, -1.f, lane);
#pragma unroll
    for (int e = 0; e < 16; ++e) C[acc_row(e, lane) * MLD + (lane & 31)] = acc[e];
  };
  int failed = 0;
#pragma unroll 1
  for (int J = 0; J < TB / SB; ++J) {
    float* rowJ = M + J * SB * MLD;
    if (w == 0) {
      // lane index laundered per sub-step: keeps the compiler from hoisting chol32's
      // 32 lane masks and LDS addresses out of the loop, which spills them
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int f = chol32(rowJ + J * SB, EJ[J & 1], gp(d.E) + J * SB * TB + J * SB, diagU + J * SB, urow, ln);
      if (failed == 0 && f) failed = J * SB + f;
    } else if (J > 0) {
      // the rest of sub-step J-1's update: blocks (I, K), I > J-1, (K <= J-1 or
      // I <= K), other than (J, J)
      const int P = J - 1;
      int q = 0;
      for (int I = J; I < TB / SB; ++I)
        for (int K = 0; K < TB / SB; ++K) {
          if ((K > P && I > K) || (I == J && K == J)) continue;
          if (q++ % 7 == w - 1) update_block(P, I, K);
        }
    }
    __syncthreads();
    if (w < 3) {  // B: M_JK <- E_JJ M_JK for the three K != J
      const int K = w < J ? w : w + 1;
      float* X = rowJ + K * SB;
      v16f acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.f;
      mma32_at(acc, EJ[J & 1], ELD, X, MLD, lane);  // sum_p E_JJ[m][p] X[p][n]
#pragma unroll
      for (int e = 0; e < 16; ++e) X[acc_row(e, lane) * MLD + (lane & 31)] = acc[e];
      if (K < J) {  // E_JK is final: block (J, K) of E (row-major, coalesced rows)
#pragma unroll
        for (int e = 0; e < 16; ++e) gp(d.E)[(J * SB + acc_row(e, lane)) * TB + K * SB + (lane & 31)] = acc[e];
      }
    }
    __syncthreads();
    if (J + 1 < TB / SB) {
      if (w == 0) update_block(J, J + 1, J + 1);  // C: what A of J+1 needs first
      __syncthreads();
    }
  }
  // U (strict upper of M, diagonal from diagU) into chol
  if (d.chol)
    for (int e = tid; e < TB * TB; e += PT) {
      const int i = e / TB, j = e % TB;
      if (i <= j && j < bk) gp(d.chol)[int64_t(k0 + i) * n + k0 + j] = i == j ? diagU[i] : M[i * MLD + j];
    }
  __syncthreads();
  // M <- E (zero above the diagonal)
  for (int e = tid; e < TB * TB / 4; e += PT) {
    const int i = e >> 5, j = 4 * (e & 31);
    float4 x = *reinterpret_cast<const float4*>(M + i * MLD + j);
    if (j > i) x.x = 0.f;
    if (j + 1 > i) x.y = 0.f;
    if (j + 2 > i) x.z = 0.f;
    if (j + 3 > i) x.w = 0.f;
    *reinterpret_cast<float4*>(M + i * MLD + j) = x;
  }
  __syncthreads();
  // P^-1 = E^T E on MFMA, upper 32x32 blocks (bi <= bj) only, mirrored: the sum
  // over p runs over the 32-row blocks kb >= bj (E is lower triangular). Block
  // costs 4 - bj, dealt so that no wave has more than 4. Each block goes straight to
  // the workspace (and its mirror), and its upper part, negated, to S_kk.
  {
    KG float* Pg = gp(d.P);
    KG float* Sk = gp(d.S) + int64_t(k0) * n + k0;
    constexpr int kBlocks[8][2] = {{0, -1}, {1, -1}, {4, -1}, {2, 3}, {5, 6}, {7, 8}, {9, -1}, {-1, -1}};
    constexpr int kBi[10] = {0, 0, 0, 0, 1, 1, 1, 2, 2, 3}, kBj[10] = {0, 1, 2, 3, 1, 2, 3, 2, 3, 3};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int qq = kBlocks[w][hh];
      if (qq < 0) continue;
      const int bi = kBi[qq], bj = kBj[qq];
      v16f acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.f;
      for (int kb = bj; kb < TB / SB; ++kb)
        mma32(acc, M + kb * SB * MLD + SB * bi, MLD, M + kb * SB * MLD + SB * bj, MLD, 1.f, lane);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = acc_row(e, lane), c = lane & 31;
        const int i = SB * bi + r, j = SB * bj + c;  // i <= j off the diagonal blocks
        Pg[i * TB + j] = acc[e];
        if (i <= j && j < bk) Sk[int64_t(i) * n + j] = -acc[e];
      }
      if (bi != bj) {  // the mirror: registers 4g..4g+3 of a lane are 4 consecutive rows i
        const int j = SB * bj + (lane & 31);
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<KG v4f*>(Pg + j * TB + SB * bi + 8 * g + 4 * (lane >> 5)) =
              v4f{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
      }
    }
  }
  if (failed && tid == 0 && *gp(d.info) == 0) *gp(d.info) = k0 + failed;
}

// Panel of step k into buffer slot `slot` (Y rows slot*TB ..). For column block
// j != k, V_j = S_kj (S_jk^T for j < k); Y_j = E V_j (the Cholesky row panel U_kj
// when j > k) goes to the panel buffer and W_j = P^-1 V_j into S in place (S_kj =
// W_j, or S_jk = W_j^T). The pivot kernel wrote S_kk = -P^-1.
// Two 512-thread blocks share a tile, each taking 64 of its 128 columns (h*64 ..):
// a block reads only its own columns of V_j and writes W back only over them, so
// neither block can overwrite what the other has still to read. The block stages its
// 128x64 half of V_j in LDS, split into three bf16 planes; waves 0-3 form Y and waves
// 4-7 W, each wave a 32x64 slab (rows 32w ..) whose A operand (U_kk^-1 = E^T or P^-1,
// read as rows of E or of the symmetric P^-1) streams from L2 into registers one 16-deep step ahead
// and is split there; every product runs as the six bf16 MFMA products of the tile
// engine (fp32 accuracy). E is lower triangular, so a Y row m only sums k <= m. Blocks b and b+8 (one XCD, so the
// second read of the A operands hits that XCD's L2) take the two halves of one tile.
// For slot >= 1, blocks from `base` on give step k-1 (panel slot-1) to the diagonal
// blocks of the group's later pivots k+1.. (block (p, u): matrix p, pivot kg+1+u),
// which nothing else in the launch reads or writes; Vs is their staging LDS.
constexpr int PP = 512;        // panel threads
constexpr int PH = TB / 2;     // columns of V_j per block
constexpr int WTP = TB + 1;    // pitch of the transposed W half in LDS
constexpr int PANEL_LDS = X3_LDS_BYTES / 4;  // floats
static_assert(PANEL_LDS * 4 >= 3 * TB * PH * 2 && PANEL_LDS >= PH * WTP, "panel LDS too small");
__global__ void __launch_bounds__(PP) __attribute__((amdgpu_waves_per_eu(4, 4)))
inv_panel_kernel(const InvDesc* __restrict__ desc, const int32_t* __restrict__ begin, int count, int k,
                 int slot, int total, int base) {
  __shared__ __attribute__((aligned(16))) float Vs[PANEL_LDS];
  const int bid = blockIdx.x;
  if (GS > 2 && bid >= base) {  // step k-1 on a later pivot's diagonal block
    constexpr int L = GS > 2 ? GS - 1 : 1;  // later pivots per matrix at most
    const int e = bid - base, p = e / L, u = e - p * L;
    if (p >= count) return;
    const InvDesc& d = desc[p];
    const int kp = k - slot + 1 + u;  // the later pivot kg+1+u
    if (kp <= k || kp >= d.ns) return;
    update_tile(d, kp, kp, (slot - 1) * TB, slot * TB, Vs);
    return;
  }
  const int t = (bid >> 4) * 8 + (bid & 7), h = (bid >> 3) & 1;
  if (t >= total) return;
  const int p = find_problem(begin, count, t);
  const InvDesc& d = desc[p];
  const int j = t - begin[p];
  if (j == k) return;
  const int n = d.n, k0 = k * TB, bk = min(TB, n - k0);
  const int c0 = h * PH;                         // first column of this half
  const int j0 = j * TB + c0, bj = min(TB, n - j * TB) - c0;  // columns [j0, j0 + bj)
  if (bj <= 0) return;  // no columns in this half
  const int tid = threadIdx.x;
  const int grp = tid >> 8, w = (tid >> 6) & 3, lane = tid & 63;
  const int ml = lane & 31, kh = lane >> 5;
  const int mr = 32 * w;  // first row of this wave's slab
  // A operand element (k, m) = U_kk^-1[k][m] = E[m][k] (Y) or P^-1[k][m] = P^-1[m][k] (W,
  // symmetric, both triangles stored with the same bits): row m of E or P^-1, so that a
  // lane's 8 values of k are 32 consecutive bytes; zero for k, m >= bk
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(grp == 0 ? d.E : d.P), 0, TB * TB * 4, 0x00020000);
  const int kmax = grp == 0 ? min(bk, mr + 32) : bk;
  const int nstep = (kmax + 15) >> 4;  // 16-deep steps, wave-uniform
  const int m = mr + ml;
  // lane (m, kh) loads A(k, m) for k = 16c + 8kh .. +7 as two 16-byte loads, one step
  // ahead of the MFMAs
  auto load_a = [&](float (&a)[8], int c) {
    const int k8 = 16 * c + 8 * kh;
    const bool ok = m < bk && c < nstep;
    const unsigned off = ok ? static_cast<unsigned>(m * TB + k8) * 4u : 0x80000000u;
    const v4f lo = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    const v4f hi = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = k8 + i < bk ? lo[i] : 0.f;
      a[4 + i] = k8 + 4 + i < bk ? hi[i] : 0.f;
    }
  };
  constexpr int PF = 2;  // steps of A loaded ahead of the products
  float abuf[PF + 1][8];
#pragma unroll
  for (int c = 0; c < PF; ++c) load_a(abuf[c], c);  // in flight together with the V loads
  // V (128 x 64) staged as three bf16 planes [k][n] (exact split, see oct_gemm), rows
  // of 64 swizzled so that the transposing operand reads are conflict-free
  __bf16* vp = reinterpret_cast<__bf16*>(Vs);
  constexpr int VPL = TB * PH;  // bf16 per plane
  auto swz = [](int kk, int nn) { return kk * PH + ((((nn >> 2) ^ (((kk >> 1) & 1) << 3))) << 2); };
  auto split3 = [](float x, __bf16& h0, __bf16& h1, __bf16& h2) {
    h0 = static_cast<__bf16>(x);
    const float r1 = x - static_cast<float>(h0);
    h1 = static_cast<__bf16>(r1);
    h2 = static_cast<__bf16>(r1 - static_cast<float>(h1));
  };
  if (j > k) {  // V[r][c] = S[k0 + r][j0 + c]: thread 4 columns 4(tid % 16).., rows tid / 16 + 32q
    const int c4 = 4 * (tid & 15), ra = tid >> 4;
    float v[4][4];
    if (bk == TB && c4 + 4 <= bj) {  // 16-byte row segments
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f4u x = *reinterpret_cast<const KG f4u*>(gp(d.S) + int64_t(k0 + ra + 32 * q) * n + j0 + c4);
#pragma unroll
        for (int u = 0; u < 4; ++u) v[q][u] = x[u];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = ra + 32 * q;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float x = gp(d.S)[int64_t(k0 + min(r, bk - 1)) * n + j0 + min(c4 + u, bj - 1)];
          v[q][u] = (r < bk && c4 + u < bj) ? x : 0.f;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v4bf p0, p1, p2;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        __bf16 h0, h1, h2;
        split3(v[q][u], h0, h1, h2);
        p0[u] = h0; p1[u] = h1; p2[u] = h2;
      }
      const int o = swz(ra + 32 * q, c4);
      *reinterpret_cast<v4bf*>(vp + o) = p0;
      *reinterpret_cast<v4bf*>(vp + VPL + o) = p1;
      *reinterpret_cast<v4bf*>(vp + 2 * VPL + o) = p2;
    }
  } else {  // V[r][c] = S[j0 + c][k0 + r]: thread the 4x4 block of rows 4(tid / 16).. and
           // columns 4(tid % 16)..; a column of V is a row of S, read 16 bytes at a time
    const int c4 = 4 * (tid & 15), r4 = 4 * (tid >> 4);
    float v[4][4];  // v[row][column]
    if (r4 + 4 <= bk && c4 + 4 <= bj) {
#pragma unroll
      for (int uc = 0; uc < 4; ++uc) {
        const f4u x = *reinterpret_cast<const KG f4u*>(gp(d.S) + int64_t(j0 + c4 + uc) * n + k0 + r4);
#pragma unroll
        for (int ur = 0; ur < 4; ++ur) v[ur][uc] = x[ur];
      }
    } else {
#pragma unroll
      for (int uc = 0; uc < 4; ++uc)
#pragma unroll
        for (int ur = 0; ur < 4; ++ur) {
          const int r = r4 + ur, c = c4 + uc;
          const float x = gp(d.S)[int64_t(j0 + min(c, bj - 1)) * n + k0 + min(r, bk - 1)];
          v[ur][uc] = (r < bk && c < bj) ? x : 0.f;
        }
    }
#pragma unroll
    for (int ur = 0; ur < 4; ++ur) {
      v4bf p0, p1, p2;
#pragma unroll
      for (int uc = 0; uc < 4; ++uc) {
        __bf16 h0, h1, h2;
        split3(v[ur][uc], h0, h1, h2);
        p0[uc] = h0; p1[uc] = h1; p2[uc] = h2;
      }
      const int o = swz(r4 + ur, c4);
      *reinterpret_cast<v4bf*>(vp + o) = p0;
      *reinterpret_cast<v4bf*>(vp + VPL + o) = p1;
      *reinterpret_cast<v4bf*>(vp + 2 * VPL + o) = p2;
    }
  }
  v16f acc0, acc1;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc0[e] = acc1[e] = 0.f;
  __syncthreads();
  // B operand (8 k of column n = lane % 32 of an n-block) from a plane: two
  // transposing reads (rows +0 and +4), as in the tile engine
  auto opnd = [&](const __bf16* plane, int c, int n0) {
    const int s16 = lane & 15;
    const int nn = n0 + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
    const int kk = 16 * c + 8 * kh + (s16 >> 2);
    const v4bf lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(plane + swz(kk, nn)));
    const v4bf hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(plane + swz(kk + 4, nn)));
    return v8bf{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  // the step loop unrolled by PF + 1 so that the register buffers are named statically
  auto step = [&](int c, float (&acur)[8], float (&anext)[8]) {
    load_a(anext, c + PF);
    v8bf a0, a1, a2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __bf16 h0, h1, h2;
      split3(acur[i], h0, h1, h2);
      a0[i] = h0; a1[i] = h1; a2[i] = h2;
    }
    v8bf b[2][3];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) b[nb][pl] = opnd(vp + pl * VPL, c, 32 * nb);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b[0][0], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b[1][0], acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b[0][1], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b[1][1], acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[0][2], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[1][2], acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b[0][0], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b[1][0], acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[0][1], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[1][1], acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[0][0], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[1][0], acc1, 0, 0, 0);
  };
  for (int c = 0; c < nstep; c += PF + 1) {
    step(c, abuf[0], abuf[2]);
    if (c + 1 < nstep) step(c + 1, abuf[1], abuf[0]);
    if (c + 2 < nstep) step(c + 2, abuf[2], abuf[1]);
  }
  // accumulator register e of block b: row mr + 8(e/4) + 4kh + e%4, column 32b + ml
  if (grp == 0) {
    KG float* Y = gp(d.Y) + int64_t(slot) * TB * d.ldy + j0;
    KG float* U = (d.chol && j > k) ? gp(d.chol) + int64_t(k0) * n + j0 : nullptr;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = mr + 8 * (e >> 2) + 4 * kh + (e & 3);
      const int ca = ml, cb = 32 + ml;
      if (r < bk) {
        if (ca < bj) Y[int64_t(r) * d.ldy + ca] = acc0[e];
        if (cb < bj) Y[int64_t(r) * d.ldy + cb] = acc1[e];
        if (U) {
          if (ca < bj) U[int64_t(r) * n + ca] = acc0[e];
          if (cb < bj) U[int64_t(r) * n + cb] = acc1[e];
        }
      }
    }
  } else if (j > k) {  // S_kj = W_j over this block's columns
    KG float* W = gp(d.S) + int64_t(k0) * n + j0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = mr + 8 * (e >> 2) + 4 * kh + (e & 3);
      const int ca = ml, cb = 32 + ml;
      if (r < bk) {
        if (ca < bj) W[int64_t(r) * n + ca] = acc0[e];
        if (cb < bj) W[int64_t(r) * n + cb] = acc1[e];
      }
    }
  }
  if (j < k) {  // S_jk = W_j^T over this block's rows of S, through LDS (pitch WTP)
    __syncthreads();  // every wave is done reading Vs
    if (grp == 1) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = mr + 8 * (e >> 2) + 4 * kh + (e & 3);
        Vs[ml * WTP + r] = acc0[e];
        Vs[(32 + ml) * WTP + r] = acc1[e];
      }
    }
    __syncthreads();
    for (int e = tid; e < PH * TB; e += PP) {
      const int c = e >> 7, r = e & (TB - 1);
      if (r < bk && c < bj) gp(d.S)[int64_t(j0 + c) * n + k0 + r] = Vs[c * WTP + r];
    }
  }
}

// Update after the group of steps kg .. kg+g-1 (g = min(GS, nb - kg) per matrix):
// a tile outside the group's block rows takes the product of all g steps; a tile in
// block row kg+s (the larger s if both of its indices are in the group) was rewritten
// by that step's panel and takes only the later steps; the last step's row is left
// as its panel wrote it.
// The last column of a matrix with a bordered last column (ns < nb) is 1 wide: it is
// not updated as tiles but by blocks from `tgrid` on, four per row block (p, j) of the
// panel enumeration (offsets pbegin, ptotal row blocks in all), each 32 rows, as a
// matrix-vector product over the same steps a tile (j, nb-1) would take: K split into
// 16 slices over the block's threads, the slices summed through LDS.
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) inv_update_kernel(const InvDesc* __restrict__ desc,
                                                         const int32_t* __restrict__ begin,
                                                         int count, int kg, int total, int tgrid,
                                                         const int32_t* __restrict__ pbegin, int ptotal) {
  __shared__ __attribute__((aligned(16))) float lds[4 * CHUNK];
  if (static_cast<int>(blockIdx.x) >= tgrid) {
    const int u = (blockIdx.x - tgrid) >> 2, part = (blockIdx.x - tgrid) & 3;
    if (u >= ptotal) return;
    const int p = find_problem(pbegin, count, u);
    const InvDesc& d = desc[p];
    if (d.ns == d.nb) return;
    const int j = u - pbegin[p];
    const int g = min(GS, d.ns - kg), last = kg + g - 1;
    const int m = (j >= kg && j <= last) ? j - kg : -1;
    if (m == g - 1) return;
    const int kb = (m + 1) * TB, ke = (g - 1) * TB + min(TB, d.n - last * TB);
    const int r = threadIdx.x & 31, q = threadIdx.x >> 5;  // row in the part, K slice
    const int64_t n = d.n, i = int64_t(j) * TB + part * 32 + r, c = n - 1;
    const KG float* Y = gp(static_cast<const float*>(d.Y));
    float acc = 0.f;
    if (i < n) {
#pragma unroll 8
      for (int t = kb + q; t < ke; t += 16) acc = fmaf(Y[int64_t(t) * d.ldy + i], Y[int64_t(t) * d.ldy + c], acc);
    }
    lds[q * 32 + r] = acc;
    __syncthreads();
    if (q == 0 && i < n) {
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) sum += lds[k * 32 + r];
      gp(d.S)[i * n + c] -= sum;
    }
    return;
  }
  const int v = xcd_virtual(blockIdx.x, tgrid, total);
  if (v < 0) return;
  const int p = find_problem(begin, count, v);
  const InvDesc& d = desc[p];
  int ti, tj;
  upper_tile(v - begin[p], d.nb, ti, tj);
  if (d.ns < d.nb && tj == d.nb - 1) return;  // the bordered column: blocks above
  const int g = min(GS, d.ns - kg), last = kg + g - 1;
  int m = -1;  // latest group step whose panel wrote this tile
  if (ti >= kg && ti <= last) m = ti - kg;
  if (tj >= kg && tj <= last) m = max(m, tj - kg);
  if (m == g - 1) return;
  const int kb = (m + 1) * TB, ke = (g - 1) * TB + min(TB, d.n - last * TB);
  update_tile(d, ti, tj, kb, ke, lds);
}

// Bordered last column (matrix m of the call when ns < nb): after the sweep's last
// update, saves v_i = S_i,n-1 (i < n-1) and the pivot p = S_n-1,n-1 into the free panel
// buffer (p at index n-1), sets info to n if p is not a positive finite number (and no
// earlier pivot failed) and writes U_n-1,n-1 = p^1/2 into chol. One block per matrix.
__global__ void __launch_bounds__(256) inv_border_kernel(const InvDesc* __restrict__ desc) {
  const InvDesc& d = desc[blockIdx.x];
  if (d.ns == d.nb) return;
  const int64_t n = d.n;
  KG float* v = gp(d.Y);
  for (int64_t i = threadIdx.x; i < n; i += 256) v[i] = gp(d.S)[i * n + n - 1];
  if (threadIdx.x == 0) {
    const float p = gp(d.S)[(n - 1) * n + n - 1];
    if (!(p > 0.f && isfinite(p)) && *gp(d.info) == 0) *gp(d.info) = static_cast<int32_t>(n);
    if (d.chol) gp(d.chol)[(n - 1) * n + n - 1] = p * rsqrtf(p);
  }
}

// inv <- -S with both triangles written (S = inv in place); with a bordered last
// column, the last step applied on the way (saved column v, pivot p, e = p^-1/2 as
// the pivot kernel forms it: y = e v, S_ij - y_i y_j for i, j < n-1, W_i = e^2 v_i on
// the border, -e^2 at the corner; the inverse is minus each). A thread takes 4
// adjacent columns of 4 rows: tiles off the diagonal, inside the matrix and left of
// the border move them as 16-byte accesses (4-byte aligned: rows of an order that
// is not a multiple of 4 start anywhere), the others entry by entry; the mirror goes
// through LDS so that its stores also run along rows.
__global__ void __launch_bounds__(256) inv_finish_kernel(const InvDesc* __restrict__ desc,
                                                         const int32_t* __restrict__ begin, int count) {
  __shared__ float s[FT][FT + 1];
  const int p = find_problem(begin, count, blockIdx.x);
  const InvDesc& d = desc[p];
  int ti, tj;
  upper_tile(blockIdx.x - begin[p], d.nb64, ti, tj);
  const int64_t n = d.n;
  const int cg = threadIdx.x & 15, r0 = threadIdx.x >> 4;  // columns 4cg.., rows r0 + 16q
  const int64_t i0 = int64_t(ti) * FT, j0 = int64_t(tj) * FT;
  const bool border = d.ns != d.nb;
  const int64_t jend = border ? n - 1 : n;  // columns of the plain part
  const bool inner = ti < tj && j0 + FT <= jend;
  constexpr int RQ = FT / 16;
  float e = 0.f, ee = 0.f, yj[4] = {0.f, 0.f, 0.f, 0.f};
  const KG float* bv = gp(static_cast<const float*>(d.Y));
  if (border) {
    e = rsqrtf(bv[n - 1]);
    ee = e * e;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j0 + 4 * cg + u < n - 1) yj[u] = e * bv[j0 + 4 * cg + u];
  }
  f4u x[RQ];
  float bi[RQ];
#pragma unroll
  for (int q = 0; q < RQ; ++q) {  // all loads first
    const int64_t i = i0 + r0 + 16 * q, j = j0 + 4 * cg;
    bi[q] = (border && i < n - 1) ? bv[i] : 0.f;
    if (inner) {
      x[q] = *reinterpret_cast<const KG f4u*>(gp(d.S) + i * n + j);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) x[q][u] = (i < n && j + u < n && i <= j + u) ? gp(d.S)[i * n + j + u] : 0.f;
    }
  }
#pragma unroll
  for (int q = 0; q < RQ; ++q) {
    const int64_t i = i0 + r0 + 16 * q, j = j0 + 4 * cg;
    f4u v;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float y = x[q][u];
      if (border) {
        if (j + u < n - 1) y = fmaf(-(e * bi[q]), yj[u], y);  // i <= j < n-1
        else y = i < n - 1 ? ee * bi[q] : -ee;                 // border column, corner
      }
      v[u] = (i < n && j + u < n && i <= j + u) ? -y : 0.f;
    }
    if (inner) {
      *reinterpret_cast<KG f4u*>(gp(d.S) + i * n + j) = v;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i < n && j + u < n && i <= j + u) gp(d.S)[i * n + j + u] = v[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) s[r0 + 16 * q][4 * cg + u] = v[u];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < RQ; ++q) {  // mirror: row j0 + r, columns i0 + 4cg ..
    const int r = r0 + 16 * q;
    const int64_t j = j0 + r, i = i0 + 4 * cg;
    if (ti < tj && j0 + FT <= n) {
      const f4u w = {s[4 * cg][r], s[4 * cg + 1][r], s[4 * cg + 2][r], s[4 * cg + 3][r]};
      *reinterpret_cast<KG f4u*>(gp(d.S) + j * n + i) = w;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i + u < n && j < n && i + u < j) gp(d.S)[j * n + i + u] = s[4 * cg + u][r];
    }
  }
}

struct InvPlan {
  std::vector<int> order;  // matrices sorted by block count, descending
  std::vector<int32_t> tile_begin, panel_begin, t64_begin;
  std::vector<int32_t> active;  // active[k] = matrices with more than k block steps
  size_t floats = 0;            // E, P, Y for all matrices
  int max_ns = 0;               // block steps of the longest sweep
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
    pl.floats += size_t(2) * TB * TB + size_t(GS) * TB * ((nn + 3) / 4 * 4);
    pl.max_ns = std::max(pl.max_ns, block_steps(nn));
  }
  pl.active.assign(pl.max_ns, 0);
  for (int q = 0; q < count; ++q) {
    const int ns = block_steps(n[pl.order[q]]);  // non-increasing in q (n descending)
    for (int k = 0; k < ns; ++k) pl.active[k] = q + 1;
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
    d.ns = block_steps(n[m]);
    d.nb64 = (n[m] + FT - 1) / FT;
    d.shift = shift[m];
    d.E = wsf + off; off += size_t(TB) * TB;
    d.P = wsf + off; off += size_t(TB) * TB;
    d.ldy = (n[m] + 3) / 4 * 4;
    d.Y = wsf + off; off += size_t(GS) * TB * d.ldy;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  TableUpload tu;
  tu.add(d_desc, desc.data(), sizeof(InvDesc) * count);
  tu.add(d_tile, pl.tile_begin.data(), sizeof(int32_t) * count);
  tu.add(d_panel, pl.panel_begin.data(), sizeof(int32_t) * count);
  tu.add(d_t64, pl.t64_begin.data(), sizeof(int32_t) * count);
  if ((st = tu.flush(s))) return st;
  // grid sizes for the active prefix [0, a): begin[a] or the grand total
  auto grid_of = [&](const std::vector<int32_t>& begin, int a, auto per) -> unsigned {
    if (a < count) return static_cast<unsigned>(begin[a]);
    return static_cast<unsigned>(begin[count - 1] + per(pl.order[count - 1]));
  };
  auto tiles_of = [&](int m) { int nb = (n[m] + TB - 1) / TB; return nb * (nb + 1) / 2; };
  auto panels_of = [&](int m) { return (n[m] + TB - 1) / TB; };
  auto t64_of = [&](int m) { int nb = (n[m] + FT - 1) / FT; return nb * (nb + 1) / 2; };
  // two panel blocks per tile, in groups of 16 blocks covering 8 tiles
  auto panel_grid = [](unsigned tiles) { return (tiles + 7) / 8 * 16; };

  bool in_place = true;
  for (int m = 0; m < count; ++m) in_place = in_place && mat[m] == inv[m];
  if (in_place) {
    KFAC_LAUNCH(K_INV_PREP, inv_damp_kernel, dim3(grid_of(pl.panel_begin, count, panels_of)), dim3(TB), 0, s,
                d_desc, d_panel, count);
    KFAC_CHECK_LAUNCH("inv_damp_kernel");
  } else {
    KFAC_LAUNCH(K_INV_PREP, inv_prep_kernel, dim3(grid_of(pl.t64_begin, count, t64_of)), dim3(256), 0, s,
                d_desc, d_t64, count);
    KFAC_CHECK_LAUNCH("inv_prep_kernel");
  }
  for (int kg = 0; kg < pl.max_ns; kg += GS) {  // steps in groups of GS
    for (int sg = 0; sg < GS && kg + sg < pl.max_ns; ++sg) {
      const int k = kg + sg, a = pl.active[k];
      const unsigned pg = grid_of(pl.panel_begin, a, panels_of);
      // pivot k; after the first step of a group, with the group's earlier steps
      // applied to block row k in the same launch
      KFAC_LAUNCH(K_INV_PIVOT, inv_pivot_kernel, dim3(sg == 0 ? a : a + pg), dim3(PT), 0, s, d_desc, d_panel, a,
                  k, sg, sg == 0 ? 0 : static_cast<int>(pg));
      KFAC_CHECK_LAUNCH("inv_pivot_kernel");
      // after the first step of a group, with step k-1 given to the later pivots'
      // diagonal blocks in the same launch
      const unsigned pb = panel_grid(pg), diag = sg >= 1 && GS > 2 ? a * (GS - 1) : 0;
      KFAC_LAUNCH(K_INV_PANEL, inv_panel_kernel, dim3(pb + diag), dim3(PP), 0, s, d_desc, d_panel, a, k, sg,
                  static_cast<int>(pg), static_cast<int>(pb));
      KFAC_CHECK_LAUNCH("inv_panel_kernel");
    }
    const int a0 = pl.active[kg];
    const unsigned ut = grid_of(pl.tile_begin, a0, tiles_of), tg = xcd_grid(ut);
    bool any_border = false;  // matrices [0, a0) with a bordered last column
    for (int q = 0; q < a0; ++q) any_border = any_border || desc[q].ns != desc[q].nb;
    const unsigned pt = any_border ? grid_of(pl.panel_begin, a0, panels_of) : 0;
    KFAC_LAUNCH(K_INV_UPDATE, inv_update_kernel, dim3(tg + 4 * pt), dim3(512), 0, s, d_desc, d_tile, a0, kg,
                static_cast<int>(ut), static_cast<int>(tg), d_panel, static_cast<int>(pt));
    KFAC_CHECK_LAUNCH("inv_update_kernel");
  }
  bool bordered = false;
  for (int q = 0; q < count; ++q) bordered = bordered || desc[q].ns != desc[q].nb;
  if (bordered) {
    KFAC_LAUNCH(K_INV_FINISH, inv_border_kernel, dim3(count), dim3(256), 0, s, d_desc);
    KFAC_CHECK_LAUNCH("inv_border_kernel");
  }
  KFAC_LAUNCH(K_INV_FINISH, inv_finish_kernel, dim3(grid_of(pl.t64_begin, count, t64_of)), dim3(256), 0, s,
              d_desc, d_t64, count);
  KFAC_CHECK_LAUNCH("inv_finish_kernel");
  return KFAC_OK;
}

extern "C" kfac_status kfac_invert_schedule(int32_t* block, int32_t* group) {
  if (!block || !group) return fail(KFAC_ERR_INVALID, "NULL pointer argument");
  *block = TB;
  *group = GS;
  return KFAC_OK;
}
