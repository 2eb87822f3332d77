// Symmetric storage conversion, batched over matrices in one launch.
// Osawa et al. (CVPR 2019), Section 1 contributions: the Kronecker factors are
// symmetric, so their upper triangle (row by row, n(n+1)/2 floats) carries them.
//
// Work item = one 64x64 tile (ti <= tj) of one matrix. Pack reads the upper tile
// rows of the full matrix and writes the matching packed row segments. Unpack
// writes the upper tile directly and, for a full symmetric result, its mirror through
// an LDS transpose, so both global writes are row-contiguous. Pure data movement,
// bit-exact. HBM-bound.
#include "common.hpp"

namespace kfac {

struct PackDesc {
  float* full;
  float* packed;
  int32_t n;
  int32_t nb;  // 64-wide tile blocks per dimension
};

constexpr int PT = 64;

__global__ void __launch_bounds__(256) pack_kernel(const PackDesc* __restrict__ desc,
                                                   const int32_t* __restrict__ begin, int count) {
  const int p = find_problem(begin, count, blockIdx.x);
  const PackDesc d = desc[p];
  int ti, tj;
  upper_tile(blockIdx.x - begin[p], d.nb, ti, tj);
  const int64_t n = d.n;
  const int c = threadIdx.x & (PT - 1);
  const int64_t j = int64_t(tj) * PT + c;
  for (int r = threadIdx.x >> 6; r < PT; r += 4) {
    const int64_t i = int64_t(ti) * PT + r;
    if (i < n && j < n && i <= j) gp(d.packed)[packed_off(i, j, n)] = gp(d.full)[i * n + j];
  }
}

// mirror = 0 writes the upper triangle only (the lower triangle of full is left as
// it was): what a consumer that reads only the upper triangle needs, at half the
// write traffic. A thread takes 4 adjacent columns of 4 rows (16 B per row and
// operand); tiles off the diagonal and inside the matrix move them as 16-byte
// accesses (4-byte aligned: packed rows and rows of an order that is not a multiple
// of 4 start anywhere), the diagonal and edge tiles entry by entry.
typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));
__global__ void __launch_bounds__(256) unpack_kernel(const PackDesc* __restrict__ desc,
                                                     const int32_t* __restrict__ begin, int count,
                                                     int mirror) {
  __shared__ float s[PT][PT + 1];
  const int p = find_problem(begin, count, blockIdx.x);
  const PackDesc d = desc[p];
  int ti, tj;
  upper_tile(blockIdx.x - begin[p], d.nb, ti, tj);
  const int64_t n = d.n;
  const int cg = threadIdx.x & 15, r0 = threadIdx.x >> 4;  // columns 4cg.., rows r0 + 16q
  const int64_t i0 = int64_t(ti) * PT, j0 = int64_t(tj) * PT;
  constexpr int RQ = PT / 16;  // rows per thread
  const bool inner = ti < tj && j0 + PT <= n;  // every entry of the tile is in the upper triangle
  f4u v[RQ];
  // all loads of a thread in flight before the first store
#pragma unroll
  for (int q = 0; q < RQ; ++q) {
    const int64_t i = i0 + r0 + 16 * q, j = j0 + 4 * cg;
    if (inner) {
      v[q] = *reinterpret_cast<const KG f4u*>(gp(d.packed) + packed_off(i, j, n));
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[q][u] = (i < n && j + u < n && i <= j + u) ? gp(d.packed)[packed_off(i, j + u, n)] : 0.f;
    }
  }
#pragma unroll
  for (int q = 0; q < RQ; ++q) {
    const int64_t i = i0 + r0 + 16 * q, j = j0 + 4 * cg;
    if (inner) {
      *reinterpret_cast<KG f4u*>(gp(d.full) + i * n + j) = v[q];
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i < n && j + u < n && i <= j + u) gp(d.full)[i * n + j + u] = v[q][u];
    }
  }
  if (!mirror) return;
#pragma unroll
  for (int q = 0; q < RQ; ++q)
#pragma unroll
    for (int u = 0; u < 4; ++u) s[r0 + 16 * q][4 * cg + u] = v[q][u];
  __syncthreads();
  // mirror: full[j][i] = full[i][j] for i < j; this thread writes row j0 + r, columns
  // i0 + 4cg ..
#pragma unroll
  for (int q = 0; q < RQ; ++q) {
    const int r = r0 + 16 * q;
    const int64_t j = j0 + r, i = i0 + 4 * cg;
    if (inner) {
      const f4u w = {s[4 * cg][r], s[4 * cg + 1][r], s[4 * cg + 2][r], s[4 * cg + 3][r]};
      *reinterpret_cast<KG f4u*>(gp(d.full) + j * n + i) = w;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i + u < n && j < n && i + u < j) gp(d.full)[j * n + i + u] = s[4 * cg + u][r];
    }
  }
}

static size_t pack_table_bytes(int count) {
  return align256(sizeof(PackDesc) * size_t(count)) + align256(sizeof(int32_t) * size_t(count));
}

}  // namespace kfac

using namespace kfac;

static kfac_status pack_validate(int32_t count, const int32_t* n) {
  if (count < 0) return fail(KFAC_ERR_INVALID, "count must be >= 0");
  if (count > 0 && !n) return fail(KFAC_ERR_INVALID, "n is NULL");
  for (int m = 0; m < count; ++m)
    if (n[m] < 1 || n[m] > (1 << 20)) return fail(KFAC_ERR_INVALID, "n[%d] = %d out of range", m, n[m]);
  return KFAC_OK;
}

extern "C" kfac_status kfac_pack_sym_workspace(int32_t count, const int32_t* n, size_t* bytes) {
  if (!bytes) return fail(KFAC_ERR_INVALID, "bytes is NULL");
  kfac_status st = pack_validate(count, n);
  if (st) return st;
  *bytes = count ? pack_table_bytes(count) : 0;
  return KFAC_OK;
}

extern "C" kfac_status kfac_pack_sym(int32_t count, const int32_t* n, float* const* full,
                                     float* const* packed, int32_t direction, void* workspace,
                                     size_t ws_bytes, void* stream) {
  kfac_status st = pack_validate(count, n);
  if (st) return st;
  if (direction < 0 || direction > 2) return fail(KFAC_ERR_INVALID, "direction must be 0, 1 or 2");
  if (count == 0) return KFAC_OK;
  if (!full || !packed) return fail(KFAC_ERR_INVALID, "full or packed is NULL");
  std::vector<PackDesc> desc(count);
  std::vector<int32_t> begin(count);
  int64_t tiles = 0;
  for (int m = 0; m < count; ++m) {
    if (!full[m] || !packed[m]) return fail(KFAC_ERR_INVALID, "matrix %d: NULL pointer", m);
    if ((reinterpret_cast<uintptr_t>(full[m]) | reinterpret_cast<uintptr_t>(packed[m])) & 3)
      return fail(KFAC_ERR_INVALID, "matrix %d: pointers must be 4-byte aligned", m);
    const int nb = (n[m] + PT - 1) / PT;
    desc[m] = {full[m], packed[m], n[m], nb};
    begin[m] = static_cast<int32_t>(tiles);
    tiles += int64_t(nb) * (nb + 1) / 2;
  }
  if (tiles >= (int64_t(1) << 31)) return fail(KFAC_ERR_INVALID, "too many tiles");
  st = check_device();
  if (st) return st;
  const size_t need = pack_table_bytes(count);
  st = check_workspace(workspace, ws_bytes, need);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver cv(workspace);
  PackDesc* d_desc = cv.take<PackDesc>(count);
  int32_t* d_begin = cv.take<int32_t>(count);
  TableUpload tu;
  tu.add(d_desc, desc.data(), sizeof(PackDesc) * count);
  tu.add(d_begin, begin.data(), sizeof(int32_t) * count);
  if ((st = tu.flush(s))) return st;
  if (direction == 0) {
    KFAC_LAUNCH(K_PACK, pack_kernel, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, s, d_desc, d_begin, count);
    KFAC_CHECK_LAUNCH("pack_kernel");
  } else {
    KFAC_LAUNCH(K_UNPACK, unpack_kernel, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, s, d_desc, d_begin, count,
                direction == 1 ? 1 : 0);
    KFAC_CHECK_LAUNCH("unpack_kernel");
  }
  return KFAC_OK;
}
