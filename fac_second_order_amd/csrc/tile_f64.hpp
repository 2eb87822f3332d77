// fp64-accumulating variant of the 512-thread tile engine: the same staging (fp32
// operand chunks [k][m] in LDS, two chunks ahead in registers) feeding
// v_mfma_f64_16x16x4f64. Products of fp32 operands are exact in fp64, so a tile
// carries no accumulation rounding however much its terms cancel.
//
// Wave w owns rows 32*(w/2) .. +32 and columns 64*(w%2) .. +64 of the 128x128 tile
// as 2 x 4 blocks of 16x16. MFMA operand layout (16x16x4): lane l supplies A[l%16][l/16]
// and B[l/16][l%16]; accumulator register r of lane l holds D[l/16 + 4r][l%16].
#pragma once
#include "tile_f32.hpp"

namespace kfac {

typedef double v4d __attribute__((ext_vector_type(4)));

struct Oct64 {
  v4d c[2][4];
};

__device__ inline void oct64_zero(Oct64& o) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) o.c[a][b] = v4d{0.0, 0.0, 0.0, 0.0};
}

// Row of accumulator register r of block (a, .), column of block (., b), this lane.
__device__ inline int oct64_row(int lane, int a, int r) {
  return 32 * ((threadIdx.x >> 6) >> 1) + 16 * a + (lane >> 4) + 4 * r;
}
__device__ inline int oct64_col(int lane, int b) { return 64 * ((threadIdx.x >> 6) & 1) + 16 * b + (lane & 15); }

// acc += As^T Bs over one staged chunk (KT values of k, 8 k-steps of 4), the LDS
// reads of a k-step issued one step ahead of its MFMAs.
__device__ inline void oct64_mma(Oct64& o, const float* As, const float* Bs) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ml = lane & 15, kq = lane >> 4;
  float a[KT / 4][2], b[KT / 4][4];
#pragma unroll
  for (int t = 0; t < KT / 4; ++t) {
    const float* ar = As + (4 * t + kq) * LDP + wm * 32 + ml;
    const float* br = Bs + (4 * t + kq) * LDP + wn * 64 + ml;
#pragma unroll
    for (int i = 0; i < 2; ++i) a[t][i] = ar[16 * i];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[t][j] = br[16 * j];
  }
#pragma unroll
  for (int t = 0; t < KT / 4; ++t)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o.c[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(a[t][i]), static_cast<double>(b[t][j]),
                                                         o.c[i][j], 0, 0, 0);
  // schedule: reads of one k-step ahead, then per k-step 8 MFMAs and the next reads
  __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
  for (int t = 0; t < KT / 4 - 1; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
}

// oct_gemm with fp64 accumulation (same pipeline, same operand forms; no sign).
template <int MA = LD_V4, int MB = LD_V4>
__device__ inline void oct64_gemm(Oct64& o, const Operand& A, const Operand& B, int K, float* lds) {
  const int npair = (K + 2 * KT - 1) / (2 * KT);
  const __amdgpu_buffer_rsrc_t rsa = op_rsrc<MA>(A);
  const __amdgpu_buffer_rsrc_t rsb = op_rsrc<MB>(B);
  auto fa = [&](int k0, float4 (&r)[2]) { oct_fetch<MA>(A, rsa, k0, r); };
  auto fb = [&](int k0, float4 (&r)[2]) { oct_fetch<MB>(B, rsb, k0, r); };
  float4 ra0[2], rb0[2], ra1[2], rb1[2];
  fa(0, ra0);
  fb(0, rb0);
  fa(KT, ra1);
  fb(KT, rb1);
  oct_stage(lds, ra0);
  oct_stage(lds + CHUNK, rb0);
  fa(2 * KT, ra0);
  fb(2 * KT, rb0);
  __syncthreads();
  auto step = [&](int c, float4 (&ra)[2], float4 (&rb)[2]) {
    const float* cur = lds + (c & 1) * 2 * CHUNK;
    oct64_mma(o, cur, cur + CHUNK);
    float* nxt = lds + ((c + 1) & 1) * 2 * CHUNK;
    oct_stage(nxt, ra);
    oct_stage(nxt + CHUNK, rb);
    fa((c + 3) * KT, ra);
    fb((c + 3) * KT, rb);
    __syncthreads();
  };
  for (int c = 0; c < 2 * npair; c += 2) {
    step(c, ra1, rb1);
    step(c + 1, ra0, rb0);
  }
}

// Tile -> global (fp32, row-major, leading dimension ld), rows < rvalid, cols < cvalid.
__device__ inline void oct64_store(const Oct64& o, float* dst, int64_t ld, int rvalid, int cvalid) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = oct64_row(lane, a, r), col = oct64_col(lane, b);
        if (row < rvalid && col < cvalid) gp(dst)[int64_t(row) * ld + col] = static_cast<float>(o.c[a][b][r]);
      }
}

// dst += alpha * tile, the sum formed in fp64 and rounded once.
__device__ inline void oct64_axpy(const Oct64& o, float* dst, int64_t ld, int rvalid, int cvalid, float alpha) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = oct64_row(lane, a, r), col = oct64_col(lane, b);
        if (row < rvalid && col < cvalid) {
          KG float* x = gp(dst) + int64_t(row) * ld + col;
          *x = static_cast<float>(fma(static_cast<double>(alpha), o.c[a][b][r], static_cast<double>(*x)));
        }
      }
}

// Transposed store through LDS (coalesced): dst[c*ld + r] = tile[r][c] for r < rvalid,
// c < cvalid. lds needs TB*LDT floats; ends with a barrier.
__device__ inline void oct64_store_t(const Oct64& o, float* dst, int64_t ld, int rvalid, int cvalid, float* lds) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        lds[oct64_col(lane, b) * LDT + oct64_row(lane, a, r)] = static_cast<float>(o.c[a][b][r]);
  __syncthreads();
  for (int e = threadIdx.x; e < TB * TB; e += 512) {
    const int c = e / TB, r = e % TB;
    if (r < rvalid && c < cvalid) gp(dst)[int64_t(c) * ld + r] = lds[c * LDT + r];
  }
  __syncthreads();
}

}  // namespace kfac
