// fp32 MFMA tile engine: a 256-thread block accumulates a 128x128 fp32 tile
// C[m][n] += sum_k A[k][m] * B[k][n] with both operands read as rows of k
// ("A^T B" form), staged through LDS in chunks of 32 k. Four waves each own a
// 64x64 quadrant made of 2x2 v_mfma_f32_32x32x2f32 blocks.
//
// MFMA lane layout (v_mfma_f32_32x32x2f32, wave64): A operand element (m, k) sits
// in lane m + 32k, B operand element (k, n) in lane n + 32k; accumulator register e
// of lane l holds row 8*(e/4) + 4*(l/32) + e%4, column l%32 of the 32x32 block.
#pragma once
#include "common.hpp"

namespace kfac {

constexpr int TB = 128;       // tile edge
constexpr int KT = 32;        // k per LDS chunk
constexpr int LDT = TB + 1;   // LDS pitch (floats)

struct Quad {
  v16f c[2][2];
};

__device__ inline void quad_zero(Quad& q) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) q.c[a][b][e] = 0.f;
}

// Row (within the 128 tile) held by accumulator register e of block (a, .) in this lane.
__device__ inline int quad_row(int wm, int a, int e, int lane) {
  return wm * 64 + a * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}
__device__ inline int quad_col(int wn, int b, int lane) { return wn * 64 + b * 32 + (lane & 31); }

// LDS chunk [KT][LDT] <- rows [k0, k0+KT) x columns [c0, c0+TB) of a row-major
// matrix (leading dimension ld); zero where k >= kvalid or column >= cvalid.
__device__ inline void stage_rows(float* lds, const float* src, int64_t ld, int k0, int kvalid,
                                  int c0, int cvalid) {
  for (int e = threadIdx.x; e < KT * TB; e += 256) {
    const int k = e / TB, c = e % TB;
    const int gk = k0 + k, gc = c0 + c;
    lds[k * LDT + c] = (gk < kvalid && gc < cvalid) ? src[int64_t(gk) * ld + gc] : 0.f;
  }
}

// Same, fp16 source widened exactly to fp32.
__device__ inline void stage_rows_h(float* lds, const _Float16* src, int64_t ld, int k0, int kvalid,
                                    int c0, int cvalid) {
  for (int e = threadIdx.x; e < KT * TB; e += 256) {
    const int k = e / TB, c = e % TB;
    const int gk = k0 + k, gc = c0 + c;
    lds[k * LDT + c] = (gk < kvalid && gc < cvalid) ? static_cast<float>(src[int64_t(gk) * ld + gc]) : 0.f;
  }
}

// LDS chunk [KT][LDT] <- transposed read: chunk[k][c] = src[(c0+c)*ld + k0+k].
__device__ inline void stage_cols(float* lds, const float* src, int64_t ld, int k0, int kvalid,
                                  int c0, int cvalid) {
  for (int e = threadIdx.x; e < KT * TB; e += 256) {
    const int c = e / KT, k = e % KT;
    const int gk = k0 + k, gc = c0 + c;
    lds[k * LDT + c] = (gk < kvalid && gc < cvalid) ? src[int64_t(gc) * ld + gk] : 0.f;
  }
}

// acc += sign * As^T Bs over one staged chunk (KT values of k).
__device__ inline void quad_mma(Quad& q, const float* As, const float* Bs, float sign) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ml = lane & 31, kh = lane >> 5;
#pragma unroll 4
  for (int k = 0; k < KT; k += 2) {
    const float* ar = As + (k + kh) * LDT + wm * 64 + ml;
    const float* br = Bs + (k + kh) * LDT + wn * 64 + ml;
    const float a0 = ar[0] * sign, a1 = ar[32] * sign;
    const float b0 = br[0], b1 = br[32];
    q.c[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, q.c[0][0], 0, 0, 0);
    q.c[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, q.c[0][1], 0, 0, 0);
    q.c[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, q.c[1][0], 0, 0, 0);
    q.c[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, q.c[1][1], 0, 0, 0);
  }
}

// Tile <-> global (row-major, leading dimension ld), rows < rvalid, cols < cvalid.
__device__ inline void quad_load(Quad& q, const float* src, int64_t ld, int rvalid, int cvalid) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = quad_row(wm, a, e, lane), c = quad_col(wn, b, lane);
        q.c[a][b][e] = (r < rvalid && c < cvalid) ? src[int64_t(r) * ld + c] : 0.f;
      }
}

__device__ inline void quad_store(const Quad& q, float* dst, int64_t ld, int rvalid, int cvalid,
                                  float scale = 1.f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = quad_row(wm, a, e, lane), c = quad_col(wn, b, lane);
        if (r < rvalid && c < cvalid) dst[int64_t(r) * ld + c] = q.c[a][b][e] * scale;
      }
}

// Transposed store: dst[c*ld + r] = tile[r][c].
__device__ inline void quad_store_t(const Quad& q, float* dst, int64_t ld, int rvalid, int cvalid) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = quad_row(wm, a, e, lane), c = quad_col(wn, b, lane);
        if (r < rvalid && c < cvalid) dst[int64_t(c) * ld + r] = q.c[a][b][e];
      }
}

// Tile -> LDS [TB][LDT] (rows r, columns c), all 128x128 entries.
__device__ inline void quad_to_lds(const Quad& q, float* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        lds[quad_row(wm, a, e, lane) * LDT + quad_col(wn, b, lane)] = q.c[a][b][e];
}

}  // namespace kfac
