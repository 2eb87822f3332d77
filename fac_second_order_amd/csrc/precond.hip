// Preconditioned gradients G^-1 dW A^-1 of many layers, two grouped launches.
// Osawa et al. (CVPR 2019), Section 3.2, eq. (6)-(7): with dW stored [d_G, d_A]
// and vec taken row by row, (G (x) A)^-1 vec(dW) = vec(G^-1 dW A^-1). Optionally the
// update of eq. (8), w <- w - lr P, in the epilogue of the second product.
//
// Both GEMMs run on the fp32 MFMA tile engine in the form C = A_rows^T B_rows, so
// every operand is read along its rows:
//   1) T^T = (G^-1 dW)^T: A operand G^-1 (symmetric, so its rows are its
//      columns), B operand dW; the tile is written transposed into the workspace.
//   2) P = T A^-1: A operand rows of T^T, B operand A^-1.
// With fp64 accumulation both products run on the fp64 MFMA engine instead (exact
// products of the fp32 operands, fp64 sums, one rounding per output element).
#include <algorithm>

#include "tile_f64.hpp"

namespace kfac {

struct GemmDesc {
  const float* A;  // A operand, read as A[k][m] (row-major, lda)
  const void* B;   // B operand, read as B[k][n] (row-major, ldb)
  float* C;        // C[m][n] (ldc), or C[n][m] when c_trans; NULL: not stored
  float* W;        // when set: W[m][n] (ldc) -= lr * tile (not with c_trans)
  float lr;
  int32_t M, N, K;
  int32_t lda, ldb, ldc;
  int32_t b_f16;
  int32_t c_trans;
  int32_t tm, tn;  // tiles along M and N
  int32_t a_mode, b_mode;  // LD_V4 / LD_F32 (fp32 operands) or LD_F16 (B fp16)
};

// MA: load form of every A operand of the launch (one instantiation per form keeps
// the register use of the common 16-byte form; the element form, with four times the
// loads in flight, gets room for two waves per SIMD instead of four).
template <int MA>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(MA == LD_V4 ? 4 : 2, 4)))
gemm_tn_kernel(const GemmDesc* __restrict__ desc, const int32_t* __restrict__ begin, int count) {
  const int p = find_problem(begin, count, blockIdx.x);
  const GemmDesc& d = desc[p];
  // column-panel major: the tiles that share a B column panel run back to back
  const int t = blockIdx.x - begin[p];
  const int mt = t % d.tm, nt = t / d.tm;
  const int m0 = mt * TB, n0 = nt * TB;
  __shared__ __attribute__((aligned(16))) float lds[4 * CHUNK];
  Oct q;
  oct_zero(q);
  const Operand A = op_rows(d.A, d.lda, d.K, m0, d.M);
  const Operand B = d.b_f16 ? op_rows_h(static_cast<const _Float16*>(d.B), d.ldb, d.K, n0, d.N)
                            : op_rows(static_cast<const float*>(d.B), d.ldb, d.K, n0, d.N);
  if (d.b_mode == LD_V4) oct_gemm<MA, LD_V4>(q, A, B, d.K, 1.f, lds);
  else if (d.b_mode == LD_F32) oct_gemm<MA, LD_F32>(q, A, B, d.K, 1.f, lds);
  else oct_gemm<MA, LD_F16>(q, A, B, d.K, 1.f, lds);
  const int rv = min(TB, d.M - m0), cv = min(TB, d.N - n0);
  if (d.c_trans) {
    oct_store_t(q, d.C + int64_t(n0) * d.ldc + m0, d.ldc, rv, cv, lds);
  } else {
    if (d.W) oct_axpy(q, d.W + int64_t(m0) * d.ldc + n0, d.ldc, rv, cv, -d.lr);
    if (d.C) oct_store(q, d.C + int64_t(m0) * d.ldc + n0, d.ldc, rv, cv);
  }
}

// The same with fp64 accumulation (its 64 accumulator registers leave room for two
// waves per SIMD).
template <int MA>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_tn64_kernel(const GemmDesc* __restrict__ desc, const int32_t* __restrict__ begin, int count) {
  const int p = find_problem(begin, count, blockIdx.x);
  const GemmDesc& d = desc[p];
  const int t = blockIdx.x - begin[p];
  const int mt = t % d.tm, nt = t / d.tm;
  const int m0 = mt * TB, n0 = nt * TB;
  __shared__ __attribute__((aligned(16))) float lds[4 * CHUNK];
  Oct64 q;
  oct64_zero(q);
  const Operand A = op_rows(d.A, d.lda, d.K, m0, d.M);
  const Operand B = d.b_f16 ? op_rows_h(static_cast<const _Float16*>(d.B), d.ldb, d.K, n0, d.N)
                            : op_rows(static_cast<const float*>(d.B), d.ldb, d.K, n0, d.N);
  if (d.b_mode == LD_V4) oct64_gemm<MA, LD_V4>(q, A, B, d.K, lds);
  else if (d.b_mode == LD_F32) oct64_gemm<MA, LD_F32>(q, A, B, d.K, lds);
  else oct64_gemm<MA, LD_F16>(q, A, B, d.K, lds);
  const int rv = min(TB, d.M - m0), cv = min(TB, d.N - n0);
  if (d.c_trans) {
    oct64_store_t(q, d.C + int64_t(n0) * d.ldc + m0, d.ldc, rv, cv, lds);
  } else {
    if (d.W) oct64_axpy(q, d.W + int64_t(m0) * d.ldc + n0, d.ldc, rv, cv, -d.lr);
    if (d.C) oct64_store(q, d.C + int64_t(m0) * d.ldc + n0, d.ldc, rv, cv);
  }
}

// Load forms of a problem's operands: 16-byte groups for fp32 operands (rows of any
// pitch, including the odd ones of d_A = 128m + 1: a group only needs 4-byte
// alignment, and one that runs past a row's end reads the next row or, past the
// buffer's range, zeros dword by dword, which reach only output rows or columns past
// the operand's last, never stored), single elements for fp16. Every operand is read
// through a raw buffer, so it must span less than 2^31 bytes (operands_fit, checked
// before anything is enqueued).
static void set_modes(GemmDesc& g) {
  g.a_mode = reinterpret_cast<uintptr_t>(g.A) % 4 == 0 ? LD_V4 : LD_F32;
  if (g.b_f16) g.b_mode = LD_F16;
  else g.b_mode = reinterpret_cast<uintptr_t>(g.B) % 4 == 0 ? LD_V4 : LD_F32;
}

// The largest operand of a layer (G^-1 or A^-1, d x d fp32; dW, d_G x d_A) spans less
// than 2^31 bytes: d_G, d_A <= 23170.
static bool operands_fit(int64_t dg, int64_t da) {
  const int64_t lim = int64_t(1) << 31;
  return dg * dg * 4 < lim && da * da * 4 < lim && dg * da * 4 < lim;
}

// One grouped product: its problems in launch order, those whose A operand has
// 16-byte groups first (stable); begin offsets restart at 0 for the others, which run
// as a second launch of the element-form instantiation.
struct Grouped {
  std::vector<GemmDesc> g;
  std::vector<int32_t> begin;
  int n_v4 = 0;
  int64_t tiles_v4 = 0, tiles_el = 0;
  bool fits() const { return tiles_v4 < (int64_t(1) << 31) && tiles_el < (int64_t(1) << 31); }
};

static Grouped group_by_a_mode(const std::vector<GemmDesc>& in) {
  Grouped r;
  for (int pass = 0; pass < 2; ++pass) {
    int64_t t = 0;
    for (const GemmDesc& x : in) {
      if ((x.a_mode == LD_V4) != (pass == 0)) continue;
      r.g.push_back(x);
      r.begin.push_back(static_cast<int32_t>(t));
      t += int64_t(x.tm) * x.tn;
    }
    (pass == 0 ? r.tiles_v4 : r.tiles_el) = t;
    if (pass == 0) r.n_v4 = static_cast<int>(r.g.size());
  }
  return r;
}

// Launches a grouped product whose tables are at desc/begin on the device.
static kfac_status launch_grouped(int kid, bool f64, const Grouped& gr, const GemmDesc* desc, const int32_t* begin,
                                  hipStream_t s, const char* what) {
  const int count = static_cast<int>(gr.g.size());
  if (gr.n_v4 > 0) {
    const dim3 grid(static_cast<unsigned>(gr.tiles_v4));
    if (f64) KFAC_LAUNCH(kid, gemm_tn64_kernel<LD_V4>, grid, dim3(512), 0, s, desc, begin, gr.n_v4);
    else KFAC_LAUNCH(kid, gemm_tn_kernel<LD_V4>, grid, dim3(512), 0, s, desc, begin, gr.n_v4);
    KFAC_CHECK_LAUNCH(what);
  }
  if (count > gr.n_v4) {
    const dim3 grid(static_cast<unsigned>(gr.tiles_el));
    const int c = count - gr.n_v4;
    if (f64) KFAC_LAUNCH(kid, gemm_tn64_kernel<LD_F32>, grid, dim3(512), 0, s, desc + gr.n_v4, begin + gr.n_v4, c);
    else KFAC_LAUNCH(kid, gemm_tn_kernel<LD_F32>, grid, dim3(512), 0, s, desc + gr.n_v4, begin + gr.n_v4, c);
    KFAC_CHECK_LAUNCH(what);
  }
  return KFAC_OK;
}

static size_t precond_ws(int count, const int32_t* dg, const int32_t* da) {
  size_t f = 0;
  for (int l = 0; l < count; ++l) f += size_t(dg[l]) * da[l];
  return 2 * align256(sizeof(GemmDesc) * count) + 2 * align256(sizeof(int32_t) * count) +
         align256(sizeof(float) * f);
}

}  // namespace kfac

using namespace kfac;

static kfac_status precond_validate(int32_t count, const int32_t* dg, const int32_t* da) {
  if (count < 0) return fail(KFAC_ERR_INVALID, "count must be >= 0");
  if (count > 0 && (!dg || !da)) return fail(KFAC_ERR_INVALID, "d_g or d_a is NULL");
  for (int l = 0; l < count; ++l)
    if (dg[l] < 1 || da[l] < 1 || dg[l] > 65536 || da[l] > 65536)
      return fail(KFAC_ERR_INVALID, "layer %d: d_g = %d, d_a = %d out of range", l, dg[l], da[l]);
  for (int l = 0; l < count; ++l)
    if (!operands_fit(dg[l], da[l]))
      return fail(KFAC_ERR_UNSUPPORTED, "layer %d: d_g = %d, d_a = %d: operands of 2^31 bytes or more", l, dg[l],
                  da[l]);
  return KFAC_OK;
}

extern "C" kfac_status kfac_precondition_workspace(int32_t count, const int32_t* d_g, const int32_t* d_a,
                                                   size_t* bytes) {
  if (!bytes) return fail(KFAC_ERR_INVALID, "bytes is NULL");
  kfac_status st = precond_validate(count, d_g, d_a);
  if (st) return st;
  *bytes = count ? precond_ws(count, d_g, d_a) : 0;
  return KFAC_OK;
}

// kfac_precondition, and with w the update of eq. (8) (out may then be NULL); the
// products accumulate in fp32 or fp64 (accum).
static kfac_status precond_impl(int32_t count, const int32_t* d_g, const int32_t* d_a,
                                const float* const* G_inv, const float* const* A_inv,
                                const void* const* grad, kfac_dtype grad_dtype, float* const* out,
                                float* const* w, float lr, kfac_dtype accum, void* workspace, size_t ws_bytes,
                                void* stream) {
  kfac_status st = precond_validate(count, d_g, d_a);
  if (st) return st;
  if (grad_dtype != KFAC_F16 && grad_dtype != KFAC_F32)
    return fail(KFAC_ERR_UNSUPPORTED, "grad dtype %d not supported", grad_dtype);
  if (accum != KFAC_F32 && accum != KFAC_F64)
    return fail(KFAC_ERR_UNSUPPORTED, "accumulation dtype %d not supported", accum);
  if (w && !(lr - lr == 0.f)) return fail(KFAC_ERR_INVALID, "lr must be finite");
  if (count == 0) return KFAC_OK;
  if (!G_inv || !A_inv || !grad || (!out && !w)) return fail(KFAC_ERR_INVALID, "NULL pointer array");
  const int esize = grad_dtype == KFAC_F16 ? 2 : 4;
  for (int l = 0; l < count; ++l) {
    float* o = out ? out[l] : nullptr;
    float* wl = w ? w[l] : nullptr;
    if (!G_inv[l] || !A_inv[l] || !grad[l] || (out && !o) || (w && !wl))
      return fail(KFAC_ERR_INVALID, "layer %d: NULL pointer", l);
    if ((reinterpret_cast<uintptr_t>(G_inv[l]) | reinterpret_cast<uintptr_t>(A_inv[l]) |
         reinterpret_cast<uintptr_t>(o) | reinterpret_cast<uintptr_t>(wl)) & 3 ||
        reinterpret_cast<uintptr_t>(grad[l]) % esize)
      return fail(KFAC_ERR_INVALID, "layer %d: misaligned pointer", l);
    if (o && o == wl) return fail(KFAC_ERR_INVALID, "layer %d: out and w are the same buffer", l);
  }
  st = check_device();
  if (st) return st;
  st = check_workspace(workspace, ws_bytes, precond_ws(count, d_g, d_a));
  if (st) return st;
  Carver cv(workspace);
  GemmDesc* d1 = cv.take<GemmDesc>(count);
  GemmDesc* d2 = cv.take<GemmDesc>(count);
  int32_t* b1 = cv.take<int32_t>(count);
  int32_t* b2 = cv.take<int32_t>(count);
  size_t f = 0;
  for (int l = 0; l < count; ++l) f += size_t(d_g[l]) * d_a[l];
  float* tt = cv.take<float>(f);
  // Problems go in decreasing K (longest tiles first), each launch in its own order.
  std::vector<int> o1(count), o2(count);
  for (int l = 0; l < count; ++l) o1[l] = o2[l] = l;
  std::stable_sort(o1.begin(), o1.end(), [&](int a, int b) { return d_g[a] > d_g[b]; });
  std::stable_sort(o2.begin(), o2.end(), [&](int a, int b) { return d_a[a] > d_a[b]; });
  std::vector<GemmDesc> x1(count), x2(count), g1(count), g2(count);
  size_t off = 0;
  for (int l = 0; l < count; ++l) {
    const int G = d_g[l], A = d_a[l];
    float* T = tt + off;  // T^T: [d_a][d_g]
    off += size_t(G) * A;
    GemmDesc x{};
    x.A = G_inv[l]; x.B = grad[l]; x.C = T;
    x.M = G; x.N = A; x.K = G;
    x.lda = G; x.ldb = A; x.ldc = G;
    x.b_f16 = grad_dtype == KFAC_F16; x.c_trans = 1;
    x.tm = (G + TB - 1) / TB; x.tn = (A + TB - 1) / TB;
    set_modes(x);
    x1[l] = x;
    GemmDesc y{};
    y.A = T; y.B = A_inv[l]; y.C = out ? out[l] : nullptr;
    y.W = w ? w[l] : nullptr; y.lr = lr;
    y.M = G; y.N = A; y.K = A;
    y.lda = G; y.ldb = A; y.ldc = A;
    y.b_f16 = 0; y.c_trans = 0;
    y.tm = x.tm; y.tn = x.tn;
    set_modes(y);
    x2[l] = y;
  }
  for (int q = 0; q < count; ++q) {
    g1[q] = x1[o1[q]];
    g2[q] = x2[o2[q]];
  }
  const Grouped p1 = group_by_a_mode(g1), p2 = group_by_a_mode(g2);
  if (!p1.fits() || !p2.fits()) return fail(KFAC_ERR_INVALID, "too many tiles");
  hipStream_t s = static_cast<hipStream_t>(stream);
  TableUpload tu;
  tu.add(d1, p1.g.data(), sizeof(GemmDesc) * count);
  tu.add(d2, p2.g.data(), sizeof(GemmDesc) * count);
  tu.add(b1, p1.begin.data(), sizeof(int32_t) * count);
  tu.add(b2, p2.begin.data(), sizeof(int32_t) * count);
  if ((st = tu.flush(s))) return st;
  const bool f64 = accum == KFAC_F64;
  const int kid = f64 ? K_GEMM64 : K_GEMM;
  if ((st = launch_grouped(kid, f64, p1, d1, b1, s, "gemm_tn kernel (G^-1 dW)"))) return st;
  if ((st = launch_grouped(kid, f64, p2, d2, b2, s, "gemm_tn kernel (T A^-1)"))) return st;
  return KFAC_OK;
}

extern "C" kfac_status kfac_precondition(int32_t count, const int32_t* d_g, const int32_t* d_a,
                                         const float* const* G_inv, const float* const* A_inv,
                                         const void* const* grad, kfac_dtype grad_dtype,
                                         float* const* out, void* workspace, size_t ws_bytes,
                                         void* stream) {
  if (count > 0 && !out) return fail(KFAC_ERR_INVALID, "NULL pointer array");
  return precond_impl(count, d_g, d_a, G_inv, A_inv, grad, grad_dtype, out, nullptr, 0.f, KFAC_F32, workspace,
                      ws_bytes, stream);
}

extern "C" kfac_status kfac_precondition_update(int32_t count, const int32_t* d_g, const int32_t* d_a,
                                                const float* const* G_inv, const float* const* A_inv,
                                                const void* const* grad, kfac_dtype grad_dtype,
                                                float* const* out, float* const* w, float lr,
                                                void* workspace, size_t ws_bytes, void* stream) {
  if (count > 0 && !w) return fail(KFAC_ERR_INVALID, "NULL weight array");
  return precond_impl(count, d_g, d_a, G_inv, A_inv, grad, grad_dtype, out, w, lr, KFAC_F32, workspace, ws_bytes,
                      stream);
}

extern "C" kfac_status kfac_precondition_ex(int32_t count, const int32_t* d_g, const int32_t* d_a,
                                            const float* const* G_inv, const float* const* A_inv,
                                            const void* const* grad, kfac_dtype grad_dtype, float* const* out,
                                            float* const* w, float lr, kfac_dtype accum, void* workspace,
                                            size_t ws_bytes, void* stream) {
  return precond_impl(count, d_g, d_a, G_inv, A_inv, grad, grad_dtype, out, w, lr, accum, workspace, ws_bytes,
                      stream);
}

// ---- refinement of a computed inverse -------------------------------------------
// One step of X <- X + X E with E = I - (F + sI) X, for inverses X of damped factors
// (the fp64-residual refinement of an approximate inverse; Osawa et al. (CVPR 2019),
// Section 3.2, eq. (6), for the inverse itself). E is formed as (I - sX) - F X: the
// product F X summed in fp64 on the fp64 engine and subtracted from the fp32 I - sX in
// its epilogue, so E carries only the roundings of I - sX and of E itself (adding s
// to F first would round F's diagonal and perturb M by far more than the residual).
// The correction X E (fp32 sums) is added symmetrised, (C + C^T) / 2.
namespace kfac {

// E <- I - s X over matrix p's elements, blocks of 1024 elements (offsets ebegin).
__global__ void __launch_bounds__(256) refine_init_kernel(const float* const* __restrict__ X, float* const* __restrict__ E,
                                                          const int32_t* __restrict__ n, const float* __restrict__ s,
                                                          const int32_t* __restrict__ ebegin, int count) {
  const int p = find_problem(ebegin, count, blockIdx.x);
  const int64_t nn = n[p], total = nn * nn;
  const int64_t e0 = int64_t(blockIdx.x - ebegin[p]) * 1024;
  for (int64_t e = e0 + threadIdx.x; e < min(total, e0 + 1024); e += 256) {
    const int64_t i = e / nn, j = e - i * nn;
    gp(E[p])[e] = (i == j ? 1.f : 0.f) - s[p] * gp(X[p])[e];
  }
}

// X <- X + (C + C^T) / 2, 64x64 tiles (offsets tbegin), the transposed tile through LDS.
__global__ void __launch_bounds__(256) refine_apply_kernel(float* const* __restrict__ X, const float* const* __restrict__ C,
                                                           const int32_t* __restrict__ n, const int32_t* __restrict__ tbegin,
                                                           int count) {
  __shared__ float t[64][65];
  const int p = find_problem(tbegin, count, blockIdx.x);
  const int64_t nn = n[p];
  const int nb = static_cast<int>((nn + 63) / 64);
  const int q = blockIdx.x - tbegin[p], ti = q / nb, tj = q - ti * nb;
  const int c = threadIdx.x & 63;
  const int64_t i0 = int64_t(ti) * 64, j0 = int64_t(tj) * 64;
  for (int r = threadIdx.x >> 6; r < 64; r += 4) {  // t[c][r] = C[j0 + r][i0 + c]
    const int64_t a = j0 + r, b = i0 + c;
    t[c][r] = (a < nn && b < nn) ? gp(C[p])[a * nn + b] : 0.f;
  }
  __syncthreads();
  for (int r = threadIdx.x >> 6; r < 64; r += 4) {
    const int64_t i = i0 + r, j = j0 + c;
    if (i < nn && j < nn) {
      const int64_t o = i * nn + j;
      gp(X[p])[o] += 0.5f * (gp(C[p])[o] + t[r][c]);
    }
  }
}

// Workspace in carve order: two descriptor tables, four offset tables, three pointer
// tables, orders and shifts, then E and C (n x n each) per matrix.
static size_t refine_ws(int count, const int32_t* n) {
  size_t f = 0;
  for (int m = 0; m < count; ++m) f += 2 * size_t(n[m]) * n[m];
  return 2 * align256(sizeof(GemmDesc) * count) + 4 * align256(sizeof(int32_t) * count) +
         3 * align256(sizeof(void*) * count) + align256(sizeof(int32_t) * count) + align256(sizeof(float) * count) +
         align256(sizeof(float) * f);
}

}  // namespace kfac

extern "C" kfac_status kfac_invert_refine_workspace(int32_t count, const int32_t* n, size_t* bytes) {
  if (!bytes) return fail(KFAC_ERR_INVALID, "bytes is NULL");
  kfac_status st = precond_validate(count, n, n);
  if (st) return st;
  *bytes = count ? refine_ws(count, n) : 0;
  return KFAC_OK;
}

extern "C" kfac_status kfac_invert_refine(int32_t count, const int32_t* n, const float* const* mat,
                                          const float* shift, float* const* inv, void* workspace,
                                          size_t ws_bytes, void* stream) {
  kfac_status st = precond_validate(count, n, n);
  if (st) return st;
  if (count == 0) return KFAC_OK;
  if (!mat || !shift || !inv) return fail(KFAC_ERR_INVALID, "NULL pointer argument");
  for (int m = 0; m < count; ++m) {
    if (!mat[m] || !inv[m]) return fail(KFAC_ERR_INVALID, "matrix %d: NULL pointer", m);
    if ((reinterpret_cast<uintptr_t>(mat[m]) | reinterpret_cast<uintptr_t>(inv[m])) & 3)
      return fail(KFAC_ERR_INVALID, "matrix %d: misaligned pointer", m);
    if (!(shift[m] - shift[m] == 0.f)) return fail(KFAC_ERR_INVALID, "matrix %d: shift is not finite", m);
  }
  {  // no inv buffer may overlap any mat or inv buffer (mat buffers are only read)
    struct Range { uintptr_t lo, hi; int m; bool out; };
    std::vector<Range> r;
    r.reserve(2 * count);
    for (int m = 0; m < count; ++m) {
      const uintptr_t bytes = uintptr_t(n[m]) * uintptr_t(n[m]) * 4;
      r.push_back({reinterpret_cast<uintptr_t>(mat[m]), reinterpret_cast<uintptr_t>(mat[m]) + bytes, m, false});
      r.push_back({reinterpret_cast<uintptr_t>(inv[m]), reinterpret_cast<uintptr_t>(inv[m]) + bytes, m, true});
    }
    std::sort(r.begin(), r.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
    // sweep in address order: each range against the furthest-reaching earlier one of
    // each kind (an overlap of two mat ranges is allowed)
    uintptr_t end_in = 0, end_out = 0;
    int m_in = -1, m_out = -1;
    for (const Range& x : r) {
      if (x.out && x.lo < end_in) return fail(KFAC_ERR_INVALID, "inv[%d] overlaps mat[%d]", x.m, m_in);
      if (x.lo < end_out) return fail(KFAC_ERR_INVALID, "%s[%d] overlaps inv[%d]", x.out ? "inv" : "mat", x.m, m_out);
      if (x.out) { if (x.hi > end_out) { end_out = x.hi; m_out = x.m; } }
      else if (x.hi > end_in) { end_in = x.hi; m_in = x.m; }
    }
  }
  st = check_device();
  if (st) return st;
  st = check_workspace(workspace, ws_bytes, refine_ws(count, n));
  if (st) return st;
  Carver cv(workspace);
  GemmDesc* d1 = cv.take<GemmDesc>(count);
  GemmDesc* d2 = cv.take<GemmDesc>(count);
  int32_t* b1 = cv.take<int32_t>(count);
  int32_t* b2 = cv.take<int32_t>(count);
  int32_t* eb = cv.take<int32_t>(count);
  int32_t* tb = cv.take<int32_t>(count);
  float** dX = cv.take<float*>(count);
  float** dE = cv.take<float*>(count);
  float** dC = cv.take<float*>(count);
  int32_t* dn = cv.take<int32_t>(count);
  float* ds = cv.take<float>(count);
  size_t f = 0;
  for (int m = 0; m < count; ++m) f += 2 * size_t(n[m]) * n[m];
  float* buf = cv.take<float>(f);
  std::vector<int> order(count);
  for (int m = 0; m < count; ++m) order[m] = m;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return n[a] > n[b]; });
  std::vector<GemmDesc> g1(count), g2(count);
  std::vector<int32_t> ebv(count), tbv(count), nv(count);
  std::vector<float*> xv(count), ev(count), cvv(count);
  std::vector<float> sv(count);
  int64_t ne = 0, nt = 0;
  size_t off = 0;
  for (int q = 0; q < count; ++q) {
    const int m = order[q], N = n[m];
    float* E = buf + off; off += size_t(N) * N;
    float* C = buf + off; off += size_t(N) * N;
    GemmDesc x{};  // E -= F X (fp64 sums): A operand F (symmetric: rows are columns)
    x.A = mat[m]; x.B = inv[m]; x.W = E; x.lr = 1.f;
    x.M = N; x.N = N; x.K = N; x.lda = N; x.ldb = N; x.ldc = N;
    x.tm = x.tn = (N + TB - 1) / TB;
    set_modes(x);
    GemmDesc y{};  // C = X E: A operand X (symmetric)
    y.A = inv[m]; y.B = E; y.C = C;
    y.M = N; y.N = N; y.K = N; y.lda = N; y.ldb = N; y.ldc = N;
    y.tm = y.tn = x.tm;
    set_modes(y);
    g1[q] = x; g2[q] = y;
    ebv[q] = static_cast<int32_t>(ne); ne += (int64_t(N) * N + 1023) / 1024;
    tbv[q] = static_cast<int32_t>(nt); nt += int64_t((N + 63) / 64) * ((N + 63) / 64);
    xv[q] = inv[m]; ev[q] = E; cvv[q] = C;
    nv[q] = N; sv[q] = shift[m];
  }
  const Grouped p1 = group_by_a_mode(g1), p2 = group_by_a_mode(g2);
  if (!p1.fits() || !p2.fits() || ne >= (int64_t(1) << 31) || nt >= (int64_t(1) << 31))
    return fail(KFAC_ERR_INVALID, "too many tiles");
  hipStream_t s = static_cast<hipStream_t>(stream);
  TableUpload tu;
  tu.add(d1, p1.g.data(), sizeof(GemmDesc) * count);
  tu.add(d2, p2.g.data(), sizeof(GemmDesc) * count);
  tu.add(b1, p1.begin.data(), sizeof(int32_t) * count);
  tu.add(b2, p2.begin.data(), sizeof(int32_t) * count);
  tu.add(eb, ebv.data(), sizeof(int32_t) * count);
  tu.add(tb, tbv.data(), sizeof(int32_t) * count);
  tu.add(dX, xv.data(), sizeof(float*) * count);
  tu.add(dE, ev.data(), sizeof(float*) * count);
  tu.add(dC, cvv.data(), sizeof(float*) * count);
  tu.add(dn, nv.data(), sizeof(int32_t) * count);
  tu.add(ds, sv.data(), sizeof(float) * count);
  if ((st = tu.flush(s))) return st;
  KFAC_LAUNCH(K_REFINE_EW, refine_init_kernel, dim3(static_cast<unsigned>(ne)), dim3(256), 0, s, dX, dE, dn, ds, eb, count);
  KFAC_CHECK_LAUNCH("refine_init_kernel");
  if ((st = launch_grouped(K_REFINE_RES, true, p1, d1, b1, s, "gemm_tn64_kernel (E -= F X)"))) return st;
  if ((st = launch_grouped(K_REFINE_CORR, false, p2, d2, b2, s, "gemm_tn_kernel (X E)"))) return st;
  KFAC_LAUNCH(K_REFINE_EW, refine_apply_kernel, dim3(static_cast<unsigned>(nt)), dim3(256), 0, s, dX, dC, dn, tb, count);
  KFAC_CHECK_LAUNCH("refine_apply_kernel");
  return KFAC_OK;
}
